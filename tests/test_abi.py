"""C-ABI tests that need no GPU: the library loads, exports every entry point
declared in include/moda.h, and rejects invalid arguments on the host before
any launch, with the documented status codes."""
import ctypes
import os
import re
import subprocess

import pytest

from transformer_attention_moda_amd import binding as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moda.h")

# Fake device pointers: never dereferenced, because every call below fails validation.
A = 0x10000          # 16-byte aligned
MIS = 0x10008        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moda_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert set(names) == set(mb.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", mb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, f"{n} not exported"
    lib = mb.load()
    for n in names:
        assert hasattr(lib, n)


def prob(**kw):
    base = dict(B=1, Hq=4, Hk=2, T=16, d=64, L=2, scale=0.125, dtype=mb.MODA_BF16, chunk=0)
    base.update(kw)
    return mb.problem(**base)


def fwd_rc(p, ptrs=None):
    q, k, v, kd, vd, o, lse = ptrs or (A,) * 7
    lib = mb.load()
    return lib.moda_fwd(ctypes.byref(p) if p is not None else None, q, k, v, kd, vd, o, lse,
                        None)


INVALID_PROBLEMS = [
    dict(B=0), dict(Hq=0), dict(Hk=0), dict(T=0), dict(T=-3), dict(Hq=5, Hk=2), dict(L=-1),
    dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(chunk=-1), dict(reserved=1), dict(B=1 << 40, T=1 << 30, Hq=1 << 20, Hk=1 << 20),
    dict(flags=2), dict(flags=-1), dict(window=-1), dict(window=3), dict(L=0, window=1),
]
UNSUPPORTED_PROBLEMS = [
    dict(d=32), dict(d=96), dict(d=256), dict(dtype=7), dict(L=mb.MODA_MAX_L + 1),
    dict(Hq=6, Hk=2), dict(Hq=64, Hk=1), dict(T=(1 << 24) + 1),
    # staging offsets across a KV group's heads reach (G-1)*T rows: 2 GiB at most
    dict(Hq=32, Hk=1, T=1 << 20), dict(Hq=2, Hk=1, T=1 << 23, d=128),
]


@pytest.mark.parametrize("kw", INVALID_PROBLEMS)
def test_fwd_invalid_problem(kw):
    assert fwd_rc(prob(**kw)) == mb.MODA_ERR_INVALID_ARGUMENT
    assert mb.load().moda_last_error().decode()


@pytest.mark.parametrize("kw", UNSUPPORTED_PROBLEMS)
def test_fwd_unsupported_problem(kw):
    assert fwd_rc(prob(**kw)) == mb.MODA_ERR_UNSUPPORTED


def test_fwd_null_problem():
    assert mb.load().moda_fwd(None, A, A, A, A, A, A, A, None) == mb.MODA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("which", range(7))
@pytest.mark.parametrize("bad", [None, MIS])
def test_fwd_bad_pointer(which, bad):
    ptrs = [A] * 7
    ptrs[which] = bad
    assert fwd_rc(prob(), ptrs) == mb.MODA_ERR_INVALID_ARGUMENT
    assert mb.load().moda_last_error().decode()


def test_fwd_null_depth_rejected_only_when_L_positive():
    assert fwd_rc(prob(L=3), (A, A, A, None, None, A, A)) == mb.MODA_ERR_INVALID_ARGUMENT
    assert fwd_rc(prob(L=0, d=32), (A, A, A, None, None, A, A)) == mb.MODA_ERR_UNSUPPORTED


def test_workspace_bytes():
    p = prob(B=2, Hq=8, Hk=4, T=100)
    n = mb.moda_bwd_workspace_bytes(p)
    rows = 2 * 8 * 100
    assert n >= 2 * rows * 4 and n % 256 == 0
    # bf16 with depth rows also carries an fp32 row of d values per query row
    assert n >= 2 * rows * 4 + rows * 64 * 4
    n0 = mb.moda_bwd_workspace_bytes(prob(B=2, Hq=8, Hk=4, T=100, L=0))
    nf = mb.moda_bwd_workspace_bytes(prob(B=2, Hq=8, Hk=4, T=100, dtype=mb.MODA_F32))
    assert 2 * rows * 4 <= n0 < 2 * rows * 4 + 256 and n0 == nf
    # A small bf16 problem (32 key blocks of 128 keys, G = 8): its key pass is split into
    # pieces whose fp32 partial dK, dV (2 x 128 keys x d floats a piece) follow the rows.
    nsplit = mb.moda_bwd_workspace_bytes(prob(Hq=8, Hk=1, T=4096, L=0))
    rows1 = 8 * 4096
    base = (2 * rows1 * 4 + 255) // 256 * 256
    assert nsplit > base and (nsplit - base) % (2 * 128 * 64 * 4) == 0
    assert nsplit - base >= 2 * 32 * 2 * 128 * 64 * 4   # at least two pieces a key block, on average
    assert mb.moda_bwd_workspace_bytes(prob(B=0)) == 0
    assert mb.load().moda_bwd_workspace_bytes(None) == 0


def bwd_rc(p, ws=0x20000, ws_bytes=1 << 30, ptrs=None):
    ptrs = ptrs or [A] * 13
    return mb.load().moda_bwd(ctypes.byref(p), *ptrs, ws, ws_bytes, None)


def test_bwd_workspace_checks():
    p = prob()
    need = mb.moda_bwd_workspace_bytes(p)
    assert bwd_rc(p, ws=None) == mb.MODA_ERR_INVALID_ARGUMENT
    assert bwd_rc(p, ws=0x20010) == mb.MODA_ERR_INVALID_ARGUMENT      # not 256-aligned
    assert bwd_rc(p, ws_bytes=need - 1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert "smaller" in mb.load().moda_last_error().decode()


@pytest.mark.parametrize("which", range(13))
def test_bwd_bad_pointer(which):
    ptrs = [A] * 13
    ptrs[which] = None
    assert bwd_rc(prob(), ptrs=ptrs) == mb.MODA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", INVALID_PROBLEMS)
def test_bwd_invalid_problem(kw):
    assert bwd_rc(prob(**kw)) == mb.MODA_ERR_INVALID_ARGUMENT


def test_pack_checks():
    lib = mb.load()
    p = prob(L=0)
    assert lib.moda_pack_depth(ctypes.byref(p), A, A, None) == mb.MODA_ERR_INVALID_ARGUMENT
    p = prob(d=4)  # 8-byte bf16 rows
    assert lib.moda_pack_depth(ctypes.byref(p), A, A, None) == mb.MODA_ERR_UNSUPPORTED
    p = prob()
    assert lib.moda_pack_depth(ctypes.byref(p), None, A, None) == mb.MODA_ERR_INVALID_ARGUMENT
    assert lib.moda_pack_depth(ctypes.byref(p), A, MIS, None) == mb.MODA_ERR_INVALID_ARGUMENT


def test_chunk_tokens_and_status_strings():
    assert mb.moda_fwd_chunk_tokens(prob(Hq=4, Hk=2, d=128)) == 128   # 256 rows at d = 128
    assert mb.moda_fwd_chunk_tokens(prob(Hq=4, Hk=2)) == 64           # 128 rows at d = 64
    assert mb.moda_fwd_chunk_tokens(prob(Hq=4, Hk=2, chunk=64)) == 64
    assert mb.moda_fwd_chunk_tokens(prob(Hq=16, Hk=4, chunk=64)) == 64
    assert mb.moda_fwd_chunk_tokens(prob(Hq=16, Hk=4, chunk=16)) == 32
    assert mb.moda_fwd_chunk_tokens(prob(dtype=mb.MODA_F32)) == 1
    assert mb.moda_fwd_chunk_tokens(prob(d=32)) == 0
    lib = mb.load()
    for code, name in [(0, "MODA_OK"), (1, "MODA_ERR_INVALID_ARGUMENT"),
                       (2, "MODA_ERR_UNSUPPORTED"), (3, "MODA_ERR_HIP")]:
        assert lib.moda_status_string(code).decode() == name


def test_binding_raises_moda_error():
    with pytest.raises(mb.ModaError) as e:
        mb._check(mb.MODA_ERR_INVALID_ARGUMENT)
    assert e.value.status == mb.MODA_ERR_INVALID_ARGUMENT


def test_timing_hook_argument_checks():
    lib = mb.load()
    assert lib.moda_timing_arm(None, 4) == mb.MODA_ERR_INVALID_ARGUMENT
    evs = (ctypes.c_void_p * 2)()
    assert lib.moda_timing_arm(evs, -1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert lib.moda_timing_arm(None, 0) == mb.MODA_OK
    assert lib.moda_timing_count() == 0
    assert lib.moda_timing_label(0) is None
    assert lib.moda_timing_label(-1) is None


def test_decode_and_append_argument_checks():
    lib = mb.load()
    p = prob(T=16, L=2)
    ws = 0x20000
    need = mb.moda_decode_workspace_bytes(p)
    assert need > 0 and need % 256 == 0
    assert mb.moda_decode_workspace_bytes(prob(dtype=mb.MODA_F32)) == 0
    dec = lambda pp, pos, wsb=1 << 30, q=A: lib.moda_decode(  # noqa: E731
        ctypes.byref(pp), pos, q, A, A, A, A, A, A, ws, wsb, None)
    assert dec(p, -1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert dec(p, 16) == mb.MODA_ERR_INVALID_ARGUMENT
    assert dec(p, 3, wsb=need - 1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert dec(p, 3, q=MIS) == mb.MODA_ERR_INVALID_ARGUMENT
    assert dec(prob(T=16, L=2, dtype=mb.MODA_F32), 3) == mb.MODA_ERR_UNSUPPORTED
    app = lambda pp, slot, t0, n, layer=A: lib.moda_depth_append(  # noqa: E731
        ctypes.byref(pp), layer, slot, t0, n, A, None)
    assert app(p, -1, 0, 1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert app(p, 2, 0, 1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert app(p, 1, 10, 7) == mb.MODA_ERR_INVALID_ARGUMENT
    assert app(p, 1, 0, 0) == mb.MODA_ERR_INVALID_ARGUMENT
    assert app(prob(L=0), 0, 0, 1) == mb.MODA_ERR_INVALID_ARGUMENT
    assert app(p, 1, 0, 1, layer=None) == mb.MODA_ERR_INVALID_ARGUMENT
    assert app(prob(d=4, dtype=mb.MODA_BF16), 0, 0, 1) == mb.MODA_ERR_UNSUPPORTED
