"""GPU parity of the decoding step and the append-mode depth cache, through the C ABI.

moda_decode (one new token at cache position pos) is compared with the oracle's row
for that token (the forward's row of the sequence that ends there), element by element;
moda_depth_append is compared bit for bit with the oracle's append and with the packer."""
import numpy as np
import pytest
import torch

import oracle
from transformer_attention_moda_amd import binding, inputs
from parity import check, host, oracle_inputs, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def cache(B, Hq, Hk, T, d, L, seed):
    w = inputs.Workload("decode", B, Hq, Hk, T, d, L, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=seed, device=DEV, names=("Q", "K", "V", "Kd", "Vd"))
    q = x.pop("Q")[:, :, seed % T].contiguous()    # the new token's queries [B, Hq, d]
    return w, q, x


def decode_check(w, q, x, pos, window=0, causal=True, tag=""):
    O, lse = binding.decode(q, x["K"], x["V"], x["Kd"], x["Vd"], w.L, pos, w.scale,
                            window=window, causal=causal)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    if causal:
        Or, lr = oracle.decode(host(q), h["K"], h["V"], h["Kd"], h["Vd"], w.L, w.scale, pos,
                               window=window)
    else:   # non-causal: every cached key, i.e. the forward's row at pos with causal off
        Q = np.zeros((w.B, w.Hq, w.T, w.d), np.uint16)
        Q[:, :, pos] = host(q)
        rows = np.array([[b, hh, pos] for b in range(w.B) for hh in range(w.Hq)])
        Or, lr = oracle.fwd_rows(Q, h["K"], h["V"], h["Kd"], h["Vd"], w.L, w.scale, rows,
                                 causal=False, window=window)
        Or, lr = Or.reshape(w.B, w.Hq, w.d), lr.reshape(w.B, w.Hq)
    name = f"decode B{w.B} Hq{w.Hq} Hk{w.Hk} T{w.T} d{w.d} L{w.L} pos{pos} W{window}{tag}"
    check(f"{name} O", to64(O), Or, "bf16")
    check(f"{name} lse", to64(lse), lr, "bf16", fp32_output=True)
    return O, lse


DECODE_SHAPES = [
    # B, Hq, Hk, T, d, L
    (1, 4, 2, 100, 128, 5),
    (2, 8, 8, 333, 64, 0),      # G = 1, no depth
    (1, 32, 1, 77, 128, 3),     # G = 32
    (3, 16, 2, 1500, 128, 40),  # G = 8, depth rows over two blocks
    (1, 2, 1, 40, 64, 1024),    # the largest L
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "B{}Hq{}Hk{}T{}d{}L{}".format(*s))
def test_decode_matches_oracle_row(shape):
    B, Hq, Hk, T, d, L = shape
    w, q, x = cache(*shape, seed=sum(shape))
    for pos in sorted({0, 31, 32, T // 2, T - 1}):
        if pos < T:
            decode_check(w, q, x, pos)
    if L > 1:
        decode_check(w, q, x, T - 2, window=1)
        decode_check(w, q, x, T // 3, window=L - 1)
    decode_check(w, q, x, T // 2, causal=False, tag=" non-causal")


def test_decode_equals_forward_row_on_the_gpu():
    """moda_decode at position pos equals moda_fwd's row pos of the sequence 0..pos (the
    same operator reached through a different split of the work)."""
    w, q, x = cache(1, 8, 4, 600, 128, 6, seed=5)
    pos = 517
    n = pos + 1
    O, lse = binding.decode(q, x["K"], x["V"], x["Kd"], x["Vd"], w.L, pos, w.scale)
    Q = torch.zeros((1, w.Hq, n, w.d), device=DEV, dtype=torch.bfloat16)
    Q[:, :, pos] = q
    Of, lf = binding.fwd(Q, x["K"][:, :, :n].contiguous(), x["V"][:, :, :n].contiguous(),
                         x["Kd"][:, :, :n * w.L].contiguous(), x["Vd"][:, :, :n * w.L].contiguous(),
                         w.L, w.scale)
    torch.cuda.synchronize()
    check("decode vs forward row O", to64(O), to64(Of[:, :, pos]), "bf16")
    check("decode vs forward row lse", to64(lse), to64(lf[:, :, pos]), "bf16", fp32_output=True)


def test_decode_at_the_64k_cache():
    """The long-sequence workload's shapes (Hq=16, Hk=8, d=128, L=24) with a 65536-token
    cache: the last position, a middle one, and a window of 4 slots."""
    w, q, x = cache(1, 16, 8, 65536, 128, 24, seed=9)
    decode_check(w, q, x, 65535)
    decode_check(w, q, x, 40000)
    decode_check(w, q, x, 65535, window=4)


def test_decode_workspace_checks():
    w, q, x = cache(1, 4, 2, 64, 128, 2, seed=3)
    p = binding.problem(1, 4, 2, 64, 128, 2)
    need = binding.moda_decode_workspace_bytes(p)
    O = torch.empty_like(q)
    lse = torch.empty((1, 4), device=DEV)
    ws = torch.empty(need, device=DEV, dtype=torch.uint8)
    with pytest.raises(binding.ModaError):
        binding.moda_decode(p, 0, q, x["K"], x["V"], x["Kd"], x["Vd"], O, lse, ws, need - 256)
    with pytest.raises(binding.ModaError):
        binding.moda_decode(p, 64, q, x["K"], x["V"], x["Kd"], x["Vd"], O, lse, ws)


@pytest.mark.parametrize("shape", [(4, 2, 3, 50, 128), (24, 1, 8, 1000, 128), (3, 2, 1, 7, 64),
                                   (5, 1, 2, 9, 96)])
def test_depth_append_builds_the_packed_cache_bitwise(shape):
    """Appending layer l into slot l for every layer equals the packer's output and the
    oracle's append, bit for bit; a ranged append touches only its rows."""
    L, B, Hk, T, d = shape
    layers = inputs.normal(shape, seed=L + T, tensor="layers_K", device=DEV)
    packed = torch.zeros((B, Hk, T * L, d), device=DEV, dtype=torch.bfloat16)
    for l in range(L):
        binding.depth_append(packed, layers[l].contiguous(), L, l)
    ref = binding.pack_depth(layers)
    torch.cuda.synchronize()
    assert torch.equal(packed.view(torch.int16), ref.view(torch.int16))
    assert np.array_equal(host(packed), oracle.pack_depth(host(layers)))
    n, t0, slot = max(1, T // 3), T // 2, L // 2
    n = min(n, T - t0)
    new = inputs.normal((B, Hk, n, d), seed=T, tensor="layers_V", device=DEV)
    before = host(packed)
    binding.depth_append(packed, new, L, slot, t0)
    torch.cuda.synchronize()
    assert np.array_equal(host(packed), oracle.depth_append(before, host(new), L, slot, t0))


def test_append_then_decode_round_trip():
    """A depth cache built token by token with moda_depth_append (as a decoder writes
    each new token's layer entries), then decoded, matches the oracle on the same rows."""
    B, Hq, Hk, T, d, L = 1, 4, 2, 48, 128, 3
    w, q, x = cache(B, Hq, Hk, T, d, L, seed=21)
    layers = {k: inputs.normal((L, B, Hk, T, d), seed=7, tensor=k, device=DEV)
              for k in ("layers_K", "layers_V")}
    Kd = torch.zeros((B, Hk, T * L, d), device=DEV, dtype=torch.bfloat16)
    Vd = torch.zeros_like(Kd)
    for t in range(T):
        for l in range(L):
            binding.depth_append(Kd, layers["layers_K"][l, :, :, t:t + 1].contiguous(), L, l, t)
            binding.depth_append(Vd, layers["layers_V"][l, :, :, t:t + 1].contiguous(), L, l, t)
    x = dict(x, Kd=Kd, Vd=Vd)
    decode_check(w, q, x, T - 1, tag=" appended cache")
    torch.cuda.synchronize()
    assert torch.equal(Kd.view(torch.int16), binding.pack_depth(layers["layers_K"]).view(torch.int16))


def test_depth_kv_cache_class_fills_the_packed_layout():
    """DepthKVCache filled one layer per slot holds exactly the packer's output for K and V,
    and the operator reads it as it reads packed tensors (bitwise equal O)."""
    L, B, Hq, Hk, T, d = 5, 1, 4, 2, 70, 128
    lk = inputs.normal((L, B, Hk, T, d), seed=31, tensor="layers_K", device=DEV)
    lv = inputs.normal((L, B, Hk, T, d), seed=31, tensor="layers_V", device=DEV)
    c = binding.DepthKVCache(B, Hk, T, L, d, device=DEV)
    for l in range(L):
        c.append(lk[l].contiguous(), lv[l].contiguous(), l)
    Kd, Vd = c.tensors()
    pk, pv = binding.pack_depth(lk), binding.pack_depth(lv)
    torch.cuda.synchronize()
    assert torch.equal(Kd.view(torch.int16), pk.view(torch.int16))
    assert torch.equal(Vd.view(torch.int16), pv.view(torch.int16))
    q = inputs.normal((B, Hq, T, d), seed=32, tensor="Q", device=DEV)
    k = inputs.normal((B, Hk, T, d), seed=32, tensor="K", device=DEV)
    v = inputs.normal((B, Hk, T, d), seed=32, tensor="V", device=DEV)
    O1 = binding.moda_attention(q, k, v, Kd, Vd, L)
    O2, _ = binding.fwd(q, k, v, pk, pv, L)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
