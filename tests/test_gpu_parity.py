"""GPU parity: libmoda (through the C ABI) against the CPU oracle, element by
element, on the same seeded inputs.

Small and medium workloads are compared in full.  The 64K-token workload, at
the size and launch configuration the benchmark times, is compared on sampled
forward rows (rows are independent, so each is exact); on exact oracle
gradients of token ranges (dQ and the depth gradients of those tokens, and
every dK, dV row of the last 4096 keys); on every dK and dV row of every KV
group under an upstream gradient that is zero outside a token set (rows with
zero upstream gradient contribute nothing, so the oracle's restricted backward
is then complete, while the kernels still walk every query tile); and on three
full-size gradient invariants of the definition per KV group."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from transformer_attention_moda_amd import binding, inputs
from parity import (check, gather_rows, host, oracle_inputs, rows_array, run_bwd, run_fwd, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W = inputs.WORKLOADS


def abs_terms(w, x, causal=True, window=0):
    """Absolute-term sums of every output (oracle.brute), for the edge-shape bound."""
    f = {k: (to64(v) if v is not None else None) for k, v in x.items()}
    return brute.abs_terms(f["Q"], f["K"], f["V"], f.get("Kd"), f.get("Vd"), f.get("dO"), w.L,
                           w.scale, causal, window)


def fwd_full_check(w, x, chunk=0, label="", edge=False, causal=True, window=0):
    O, lse = run_fwd(x, w, chunk, causal, window)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    Or, lr = oracle.fwd(h["Q"], h["K"], h["V"], h.get("Kd"), h.get("Vd"), w.L, w.scale,
                        causal, window)
    A = abs_terms(w, x, causal, window) if edge else {}
    check(f"{w.name}{label} O", to64(O), Or, w.dtype, edge=edge, terms=A.get("O"))
    check(f"{w.name}{label} lse", to64(lse), lr, w.dtype, edge=edge, fp32_output=True)
    return O, lse


def bwd_full_check(w, x, O, lse, chunk=0, label="", edge=False, causal=True, window=0):
    dQ, dK, dV, dKd, dVd = run_bwd(x, w, O, lse, chunk, causal, window)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    g = oracle.bwd(h["Q"], h["K"], h["V"], h.get("Kd"), h.get("Vd"), h["dO"], w.L, w.scale,
                   causal, window)
    got = {"dQ": dQ, "dK": dK, "dV": dV}
    if w.L > 0:
        got.update(dKd=dKd, dVd=dVd)
    A = abs_terms(w, x, causal, window) if edge else {}
    for k, v in got.items():
        check(f"{w.name}{label} {k}", to64(v), g[k], w.dtype, edge=edge, terms=A.get(k))


# ---------------- the five workloads ----------------

def test_tiny_fp32_forward_and_backward():
    w = W["tiny_fp32"]
    x = inputs.make(w, seed=1, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = fwd_full_check(w, x)
    bwd_full_check(w, x, O, lse)


def test_small_model_forward_full():
    w = W["small_model"]
    x = inputs.make(w, seed=2, device=DEV)
    fwd_full_check(w, x)


def test_layer_1p5b_forward_one_kv_group_and_no_depth_path():
    w = W["layer_1p5b_8k"]
    x = inputs.make(w, seed=3, device=DEV)
    h = oracle_inputs(x)
    G, kv = w.G, 2
    rows = rows_array(1, w.Hq, range(w.T), heads=range(kv * G, (kv + 1) * G))
    for L in (w.L, 0):
        O, lse = binding.fwd(x["Q"], x["K"], x["V"], x["Kd"] if L else None,
                             x["Vd"] if L else None, L, w.scale)
        torch.cuda.synchronize()
        Or, lr = oracle.fwd_rows(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], L, w.scale, rows)
        check(f"{w.name} L={L} O (kv group {kv})", gather_rows(O, rows), Or, w.dtype)
        check(f"{w.name} L={L} lse (kv group {kv})", gather_rows(lse, rows)[:, None],
              lr[:, None], w.dtype, fp32_output=True)


def long_rows(w):
    T = w.T
    tokens = set(range(64)) | set(range(T - 64, T)) | set(np.linspace(0, T - 1, 48).astype(int))
    for c in (1, 7, 100, 255, 256, 511):
        for dt in (-1, 0, 1):
            t = c * 128 + dt
            if 0 <= t < T:
                tokens.add(t)
    return sorted(tokens)


def test_long_64k_forward_sampled_rows():
    w = W["long_64k"]
    x = inputs.make(w, seed=4, device=DEV)
    O, lse = run_fwd(x, w)
    torch.cuda.synchronize()
    rows = rows_array(1, w.Hq, long_rows(w))
    h = oracle_inputs(x)
    Or, lr = oracle.fwd_rows(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], w.L, w.scale, rows)
    check(f"{w.name} O ({len(rows)} sampled rows)", gather_rows(O, rows), Or, w.dtype)
    check(f"{w.name} lse ({len(rows)} sampled rows)", gather_rows(lse, rows)[:, None],
          lr[:, None], w.dtype, fp32_output=True)


@pytest.fixture(scope="module")
def long64k():
    """The 64K workload's inputs (seed 6), its forward, and exact host copies."""
    w = W["long_64k"]
    x = inputs.make(w, seed=6, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = run_fwd(x, w)
    torch.cuda.synchronize()
    yield w, x, O, lse, oracle_inputs(x)
    del x, O, lse
    torch.cuda.empty_cache()


def invariant_residuals(w, x, grads, b, kv):
    """The three gradient identities of the definition for KV group (b, kv), in fp64 on the
    device: (sum dK + sum dKd, sum dV + sum dVd - sum dO, <Q,dQ> - <K,dK> - <Kd,dKd>), each
    with the scale of the terms that make it up (the root sum of squares of the summed
    elements, or of the elementwise products)."""
    dQ, dK, dV, dKd, dVd = grads
    G = w.G
    hs = slice(kv * G, (kv + 1) * G)
    f = lambda t: t.double()  # noqa: E731
    sk = f(dK[b, kv]).sum(0) + f(dKd[b, kv]).sum(0)
    nk = (f(dK[b, kv]).square().sum(0) + f(dKd[b, kv]).square().sum(0)).sqrt()
    sv = f(dV[b, kv]).sum(0) + f(dVd[b, kv]).sum(0) - f(x["dO"][b, hs]).sum((0, 1))
    nv = (f(dV[b, kv]).square().sum(0) + f(dVd[b, kv]).square().sum(0)).sqrt()
    pq = f(x["Q"][b, hs]) * f(dQ[b, hs])
    pk = f(x["K"][b, kv]) * f(dK[b, kv])
    pd = f(x["Kd"][b, kv]) * f(dKd[b, kv])
    sp = pq.sum() - pk.sum() - pd.sum()
    npp = (pq.square().sum() + pk.square().sum() + pd.square().sum()).sqrt()
    return [(n, r.cpu().numpy(), s.cpu().numpy()) for n, r, s in
            (("sum dK + sum dKd", sk, nk), ("sum dV + sum dVd - sum dO", sv, nv),
             ("<Q,dQ> - <K,dK> - <Kd,dKd>", sp, npp))]


def test_long_64k_backward_exact_ranges_and_invariants(long64k):
    """The timed step's backward at its full size and launch configuration.
    Exact oracle gradients: for KV group (b, kv) and tokens [t_lo, t_hi) the oracle's dQ
    rows and the depth rows' dKd, dVd are complete; with t_hi = T the dK and dV rows at or
    after t_lo are complete too (only those tokens' queries see them): the last 4096 keys.
    Full size, every KV group: the identities of the definition
      sum_j dK_j + sum_r dKd_r = 0        (shifting every key by one vector shifts each
                                           row's scores by a constant),
      sum_j dV_j + sum_r dVd_r = sum dO   (adding one vector to every value adds it to
                                           every output),
      <Q,dQ> = <K,dK> + <Kd,dKd>          (scaling queries by c and keys by 1/c changes
                                           no score).
    Tolerance: if every element's error is independent with an RMS within the parity bar's
    relative Frobenius bound eps = 1e-2 of the values' RMS, a sum's error has standard
    deviation at most eps times the root sum of squares of its terms; six such deviations
    are allowed."""
    w, x, O, lse, h = long64k
    dQ, dK, dV, dKd, dVd = run_bwd(x, w, O, lse)
    torch.cuda.synchronize()
    G, T, L = w.G, w.T, w.L
    for b, kv, t_lo, t_hi in ((0, 0, T - 4096, T), (0, 5, 30000, 30024), (0, 7, 0, 24)):
        g = oracle.bwd_group(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], h["dO"], L, w.scale,
                             b, kv, t_lo, t_hi)
        hs, ts = slice(kv * G, (kv + 1) * G), slice(t_lo, t_hi)
        tag = f"{w.name} (b={b}, kv={kv}, tokens {t_lo}..{t_hi - 1})"
        check(f"{tag} dQ", to64(dQ[b, hs, ts]), g["dQ"], w.dtype)
        check(f"{tag} dKd", to64(dKd[b, kv, t_lo * L:t_hi * L]), g["dKd"], w.dtype)
        check(f"{tag} dVd", to64(dVd[b, kv, t_lo * L:t_hi * L]), g["dVd"], w.dtype)
        if t_hi == T:
            check(f"{tag} dK", to64(dK[b, kv, t_lo:]), g["dK"][t_lo:], w.dtype)
            check(f"{tag} dV", to64(dV[b, kv, t_lo:]), g["dV"][t_lo:], w.dtype)
    eps = 1e-2
    for kv in range(w.Hk):
        for name, r, scale in invariant_residuals(w, x, (dQ, dK, dV, dKd, dVd), 0, kv):
            tol = 6 * eps * scale
            used = float(np.max(np.abs(r) / tol))
            print(f"{w.name} kv={kv} {name}: max |residual| {np.max(np.abs(r)):.3e}, "
                  f"{100 * used:.1f}% of the tolerance", flush=True)
            assert used <= 1.0, (kv, name)


def sparse_tokens(T):
    """Tokens of the sparse upstream gradient: both ends, spread points and query-tile
    boundaries, so that every key block's walk meets nonzero rows early and late."""
    tok = set(range(8)) | set(range(T - 8, T)) | set(np.linspace(0, T - 1, 64).astype(int))
    for c in (1, 255, 256, 300, 511):
        tok |= {c * 128 - 1, c * 128}
    return np.array(sorted(t for t in tok if 0 <= t < T))


def test_long_64k_backward_every_key_gradient_under_sparse_upstream(long64k):
    """dO zero outside a token set S: rows outside S contribute exactly nothing to any
    gradient (dS = p (dO.v - D) and p dO vanish; D = <dO, O> = 0), on the GPU as in exact
    arithmetic.  The kernels still walk every query tile, so every dK and dV row of every KV
    group -- including the key blocks that walk all 131072 folded query rows -- is compared
    with the oracle's complete restricted backward, along with dQ and the depth gradients of
    S (the depth rows of other tokens must be exactly zero)."""
    w, x, O, lse, h = long64k
    G, T, L = w.G, w.T, w.L
    S = sparse_tokens(T)
    dO = torch.zeros_like(x["dO"])
    idx = torch.from_numpy(S).to(DEV)
    dO[:, :, idx] = x["dO"][:, :, idx]
    xs = dict(x, dO=dO)
    dQ, dK, dV, dKd, dVd = run_bwd(xs, w, O, lse)
    torch.cuda.synchronize()
    hdO = host(dO)
    rows = (torch.from_numpy(S)[:, None] * L + torch.arange(L)[None, :]).reshape(-1).to(DEV)
    other = torch.ones(T * L, dtype=torch.bool, device=DEV)
    other[rows] = False
    for kv in range(w.Hk):
        g = oracle.bwd_tokens(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], hdO, L, w.scale, 0, kv,
                              S)
        hs = slice(kv * G, (kv + 1) * G)
        tag = f"{w.name} sparse dO ({len(S)} tokens) kv={kv}"
        check(f"{tag} dK (all {T} keys)", to64(dK[0, kv]), g["dK"], w.dtype)
        check(f"{tag} dV (all {T} keys)", to64(dV[0, kv]), g["dV"], w.dtype)
        check(f"{tag} dQ", to64(dQ[0, hs][:, idx]), g["dQ"], w.dtype)
        check(f"{tag} dKd", to64(dKd[0, kv, rows]), g["dKd"], w.dtype)
        check(f"{tag} dVd", to64(dVd[0, kv, rows]), g["dVd"], w.dtype)
        assert not torch.any(dKd[0, kv, other] != 0) and not torch.any(dVd[0, kv, other] != 0)
        assert not torch.any(dQ[0, hs][:, ~torch.isin(torch.arange(T, device=DEV), idx)] != 0)


def test_million_token_sequence_sampled():
    """T = 2^20 tokens (G = 2, d = 64, L = 4), 16 times the bench length: the kernels' row
    and offset arithmetic far past the five workloads, against sampled forward rows and the
    oracle's exact gradients of the last 16 tokens (both query heads; all their depth rows,
    and the dK, dV rows only those tokens' queries see)."""
    w = inputs.Workload("t1m", B=1, Hq=2, Hk=1, T=1 << 20, d=64, L=4, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=7, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = run_fwd(x, w)
    dQ, dK, dV, dKd, dVd = run_bwd(x, w, O, lse)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    T, L, n = w.T, w.L, 16
    tokens = [0, 1, 63, 64, 127, 128, 4095, 65535, 65536, (1 << 19) - 1, 1 << 19, T - 2, T - 1]
    rows = rows_array(1, w.Hq, tokens)
    Or, lr = oracle.fwd_rows(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], L, w.scale, rows)
    check(f"{w.name} O ({len(rows)} sampled rows)", gather_rows(O, rows), Or, w.dtype)
    check(f"{w.name} lse ({len(rows)} sampled rows)", gather_rows(lse, rows)[:, None],
          lr[:, None], w.dtype, fp32_output=True)
    g = oracle.bwd_group(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], h["dO"], L, w.scale, 0, 0,
                         T - n, T)
    tag = f"{w.name} (tokens {T - n}..{T - 1})"
    check(f"{tag} dQ", to64(dQ[0, :, T - n:]), g["dQ"], w.dtype)
    check(f"{tag} dK", to64(dK[0, 0, T - n:]), g["dK"][T - n:], w.dtype)
    check(f"{tag} dV", to64(dV[0, 0, T - n:]), g["dV"][T - n:], w.dtype)
    check(f"{tag} dKd", to64(dKd[0, 0, (T - n) * L:]), g["dKd"], w.dtype)
    check(f"{tag} dVd", to64(dVd[0, 0, (T - n) * L:]), g["dVd"], w.dtype)


def test_train_4k_forward_backward_two_kv_groups():
    w = W["train_4k"]
    x = inputs.make(w, seed=5, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = run_fwd(x, w)
    dQ, dK, dV, dKd, dVd = run_bwd(x, w, O, lse)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    G = w.G
    for b, kv in ((0, 0), (3, 7)):
        g = oracle.bwd_group(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], h["dO"], w.L, w.scale,
                             b, kv)
        hs = slice(kv * G, (kv + 1) * G)
        tag = f"{w.name} (b={b}, kv={kv})"
        check(f"{tag} O", to64(O[b, hs]), g["O"], w.dtype)
        check(f"{tag} lse", to64(lse[b, hs]), g["lse"], w.dtype, fp32_output=True)
        check(f"{tag} dQ", to64(dQ[b, hs]), g["dQ"], w.dtype)
        check(f"{tag} dK", to64(dK[b, kv]), g["dK"], w.dtype)
        check(f"{tag} dV", to64(dV[b, kv]), g["dV"], w.dtype)
        check(f"{tag} dKd", to64(dKd[b, kv]), g["dKd"], w.dtype)
        check(f"{tag} dVd", to64(dVd[b, kv]), g["dVd"], w.dtype)


# ---------------- edge cases (full oracle) ----------------

EDGE = [
    # B, Hq, Hk, T, d, L
    (1, 2, 1, 1, 64, 3),        # a single token
    (1, 4, 2, 77, 128, 0),      # no depth, ragged T
    (2, 8, 8, 130, 64, 1),      # G = 1
    (1, 32, 1, 50, 128, 2),     # G = 32: one token per wave
    (1, 16, 2, 333, 128, 7),    # G = 8, ragged
    (1, 4, 1, 257, 64, 5),      # G = 4, one past a tile
    (1, 2, 2, 64, 128, 1),      # exactly one tile
    (2, 4, 2, 300, 128, 24),    # chunk boundaries inside tokens of the depth blocks
    (1, 2, 1, 33, 64, 40),      # a token's depth rows span two 32-row blocks
    (1, 4, 4, 20, 128, 64),     # G = 1, each token exactly two depth blocks
    (1, 2, 1, 5, 64, 1024),     # the largest L
    (1, 1, 1, 300, 64, 1),      # d = 64 with 8-wave workgroups, one depth row per token
]


@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "B{}Hq{}Hk{}T{}d{}L{}".format(*s))
@pytest.mark.parametrize("chunk", [0, 16])
def test_edge_shapes_forward_backward(shape, chunk):
    B, Hq, Hk, T, d, L = shape
    w = inputs.Workload("edge", B, Hq, Hk, T, d, L, chunk=chunk, dtype="bf16")
    x = inputs.make(w, seed=sum(shape) + chunk, device=DEV,
                    names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = fwd_full_check(w, x, chunk, label=f" {shape} c{chunk}", edge=True)
    bwd_full_check(w, x, O, lse, chunk, label=f" {shape} c{chunk}", edge=True)


@pytest.mark.parametrize("shape", [(1, 4, 2, 37, 64, 3), (2, 2, 1, 65, 128, 0),
                                   (1, 8, 2, 20, 128, 9)])
def test_fp32_edge_shapes(shape):
    B, Hq, Hk, T, d, L = shape
    w = inputs.Workload("edge_f32", B, Hq, Hk, T, d, L, chunk=0, dtype="f32")
    x = inputs.make(w, seed=7 + T, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = fwd_full_check(w, x)
    bwd_full_check(w, x, O, lse)


# ---------------- invariants on the GPU ----------------

def test_chunk_size_does_not_change_the_result():
    w = W["small_model"]
    x = inputs.make(w, seed=8, device=DEV)
    O1, l1 = run_fwd(x, w, chunk=64)     # 128 folded rows per workgroup
    O2, l2 = run_fwd(x, w, chunk=128)    # 256 folded rows per workgroup
    torch.cuda.synchronize()
    assert binding.moda_fwd_chunk_tokens(binding.problem_for(x["Q"], x["K"], w.L, chunk=64)) \
        != binding.moda_fwd_chunk_tokens(binding.problem_for(x["Q"], x["K"], w.L, chunk=128))
    check("chunk 64 vs 128 O", to64(O1), to64(O2), "bf16")
    check("chunk 64 vs 128 lse", to64(l1), to64(l2), "bf16")


def test_depth_slot_permutation_invariance():
    w = inputs.Workload("perm", 1, 8, 4, 500, 128, 6, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=9, device=DEV)
    perm = torch.randperm(w.L, generator=torch.Generator().manual_seed(3))
    idx = (torch.arange(w.T)[:, None] * w.L + perm[None, :]).reshape(-1).to(DEV)
    xp = dict(x, Kd=x["Kd"][:, :, idx].contiguous(), Vd=x["Vd"][:, :, idx].contiguous())
    O1, l1 = run_fwd(x, w)
    O2, l2 = run_fwd(xp, w)
    torch.cuda.synchronize()
    check("depth-permuted O", to64(O2), to64(O1), "bf16")
    check("depth-permuted lse", to64(l2), to64(l1), "bf16")


def test_sequence_to_minus_infinity_gives_depth_attention():
    # Q_t = a e1 + q', K_j = -a e1 + k', depth keys orthogonal to e1; a = 32 is exact in bf16.
    w = inputs.Workload("seqinf", 1, 4, 2, 300, 128, 5, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=10, device=DEV)
    x["Q"][..., 0] = 32.0
    x["K"][..., 0] = -32.0
    x["Kd"][..., 0] = 0.0
    O, lse = run_fwd(x, w)
    torch.cuda.synchronize()
    q = to64(x["Q"])[0]
    kd = to64(x["Kd"])[0]
    vd = to64(x["Vd"])[0]
    ref = np.zeros((w.Hq, w.T, w.d))
    for h in range(w.Hq):
        kv = h // w.G
        u = np.einsum("tld,td->tl", kd[kv].reshape(w.T, w.L, w.d), q[h]) * w.scale
        p = np.exp(u - u.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ref[h] = np.einsum("tl,tld->td", p, vd[kv].reshape(w.T, w.L, w.d))
    check("sequence at -inf: O equals depth-only attention", to64(O)[0], ref, "bf16")


def test_forward_is_deterministic():
    w = W["small_model"]
    x = inputs.make(w, seed=11, device=DEV)
    O1, l1 = run_fwd(x, w)
    O2, l2 = run_fwd(x, w)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_outputs_stay_inside_their_buffers():
    w = inputs.Workload("canary", 1, 4, 2, 157, 128, 3, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=12, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    pad = 4096
    guard = -12345.0

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), guard, device=DEV, dtype=dtype)
        return buf, buf[pad:pad + n].view(shape)

    ob, O = guarded(x["Q"].shape, torch.bfloat16)
    lb, lse = guarded(x["Q"].shape[:3], torch.float32)
    p = binding.problem_for(x["Q"], x["K"], w.L, w.scale)
    binding.moda_fwd(p, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], O, lse)
    grads = [guarded(x[k].shape, torch.bfloat16) for k in ("Q", "K", "V", "Kd", "Vd")]
    ws = torch.empty(binding.moda_bwd_workspace_bytes(p), device=DEV, dtype=torch.uint8)
    binding.moda_bwd(p, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], O, lse, x["dO"],
                     *[g[1] for g in grads], ws)
    torch.cuda.synchronize()
    for buf in [ob, lb] + [g[0] for g in grads]:
        assert torch.all(buf[:pad] == guard) and torch.all(buf[-pad:] == guard)


# ---------------- variants: non-causal, sliding-window depth ----------------

VARIANT_SHAPES = [
    # B, Hq, Hk, T, d, L
    (1, 4, 2, 77, 128, 5),      # ragged T
    (2, 8, 8, 130, 64, 3),      # G = 1
    (1, 32, 1, 50, 128, 2),     # G = 32
    (1, 16, 2, 333, 128, 7),    # G = 8, ragged
    (1, 2, 1, 33, 64, 40),      # a token's depth rows span two 32-row blocks
]
VARIANTS = [(False, 0), (True, 1), (True, -1), (False, 2)]   # (causal, window); -1: L - 1


@pytest.mark.parametrize("shape", VARIANT_SHAPES, ids=lambda s: "B{}Hq{}Hk{}T{}d{}L{}".format(*s))
@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: f"causal{int(v[0])}-W{v[1]}")
@pytest.mark.parametrize("chunk", [0, 16])
def test_variant_shapes_forward_backward(shape, variant, chunk):
    """Non-causal MoDA (every sequence key visible; the depth matching mask kept) and the
    sliding-window depth slots (the last W of L), forward and all five gradients against
    the oracle in full."""
    B, Hq, Hk, T, d, L = shape
    causal, W = variant
    W = L - 1 if W < 0 else min(W, L)
    w = inputs.Workload("variant", B, Hq, Hk, T, d, L, chunk=chunk, dtype="bf16")
    x = inputs.make(w, seed=sum(shape) + 3 * W + int(causal), device=DEV,
                    names=("Q", "K", "V", "Kd", "Vd", "dO"))
    tag = f" {shape} causal={causal} W={W} c{chunk}"
    O, lse = fwd_full_check(w, x, chunk, label=tag, edge=True, causal=causal, window=W)
    bwd_full_check(w, x, O, lse, chunk, label=tag, edge=True, causal=causal, window=W)


@pytest.mark.parametrize("variant", [(False, 0), (True, 2), (False, 1)])
def test_fp32_variants(variant):
    causal, W = variant
    w = inputs.Workload("variant_f32", 1, 4, 2, 37, 64, 3, chunk=0, dtype="f32")
    x = inputs.make(w, seed=50 + W, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = fwd_full_check(w, x, causal=causal, window=W, label=f" causal={causal} W={W}")
    bwd_full_check(w, x, O, lse, causal=causal, window=W, label=f" causal={causal} W={W}")


def test_noncausal_small_model_forward_full_and_two_kv_groups_backward():
    """The small-model workload (T = 2048, G = 2, d = 64, L = 16) without the sequence
    causal mask, at the plain bound: the whole forward, and all five gradients of two KV
    groups."""
    w = W["small_model"].with_(bwd=True)
    x = inputs.make(w, seed=13, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = fwd_full_check(w, x, label=" non-causal", causal=False)
    dQ, dK, dV, dKd, dVd = run_bwd(x, w, O, lse, causal=False)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    G = w.G
    for b, kv in ((0, 0), (1, 7)):
        g = oracle.bwd_group(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], h["dO"], w.L, w.scale,
                             b, kv, causal=False)
        hs = slice(kv * G, (kv + 1) * G)
        tag = f"{w.name} non-causal (b={b}, kv={kv})"
        for name, got in (("dQ", dQ[b, hs]), ("dK", dK[b, kv]), ("dV", dV[b, kv]),
                          ("dKd", dKd[b, kv]), ("dVd", dVd[b, kv])):
            check(f"{tag} {name}", to64(got), g[name], w.dtype)


def test_window_layer_1p5b_forward_one_kv_group():
    """The 1.5B-like layer (T = 8192, G = 4, d = 128, L = 32) seeing only the last 8 depth
    slots: one full KV group of the forward at the plain bound."""
    w = W["layer_1p5b_8k"]
    x = inputs.make(w, seed=14, device=DEV)
    O, lse = run_fwd(x, w, window=8)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    kv = 1
    rows = rows_array(1, w.Hq, range(w.T), heads=range(kv * w.G, (kv + 1) * w.G))
    Or, lr = oracle.fwd_rows(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], w.L, w.scale, rows,
                             window=8)
    check(f"{w.name} W=8 O (kv group {kv})", gather_rows(O, rows), Or, w.dtype)
    check(f"{w.name} W=8 lse (kv group {kv})", gather_rows(lse, rows)[:, None], lr[:, None],
          w.dtype, fp32_output=True)


# ---------------- depth packer ----------------

@pytest.mark.parametrize("shape", [(3, 1, 2, 5, 128), (24, 2, 3, 77, 64), (1, 1, 1, 1, 128),
                                   (32, 1, 8, 512, 128), (5, 2, 1, 9, 96)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_depth_is_an_exact_transpose(shape, dtype):
    L, B, Hk, T, d = shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    layers = inputs.normal(shape, seed=L + T, tensor="layers_K", device=DEV, dtype=tdt)
    packed = binding.pack_depth(layers)
    torch.cuda.synchronize()
    assert np.array_equal(host(packed), oracle.pack_depth(host(layers)))
