"""GPU parity at the pages' own kernel workloads (README "Kernel Efficiency": the sequence
length, GQA group and depth sweeps at d=64, Hk=8; the paper summary's Table 7 ablation
shape), in the launch configuration the benchmark suite times: sampled forward rows (rows
are independent, so each is exact) and the exact gradients of the last 48 tokens of one KV
group (their dQ rows and depth rows, and the dK, dV rows only they see).  And the depth-row
scan ablation: every scan gives the operator's result."""
import numpy as np
import pytest
import torch

import oracle
from transformer_attention_moda_amd import binding, inputs
from parity import check, gather_rows, oracle_inputs, rows_array, run_bwd, run_fwd, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PW = inputs.PAGE_WORKLOADS


@pytest.mark.parametrize("name", sorted(PW))
def test_page_workload_sampled_rows_and_exact_gradient_range(name):
    w = PW[name]
    x = inputs.make(w, seed=60, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = run_fwd(x, w)
    dQ, dK, dV, dKd, dVd = run_bwd(x, w, O, lse)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    G, T, L = w.G, w.T, w.L
    tokens = sorted(set(range(8)) | set(range(T - 8, T)) | set(np.linspace(0, T - 1, 8).astype(int)))
    rows = rows_array(1, w.Hq, tokens, heads=[0, G - 1, 3 * G, w.Hq - 1])
    Or, lr = oracle.fwd_rows(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], L, w.scale, rows)
    check(f"{name} O ({len(rows)} sampled rows)", gather_rows(O, rows), Or, w.dtype)
    check(f"{name} lse ({len(rows)} sampled rows)", gather_rows(lse, rows)[:, None], lr[:, None],
          w.dtype, fp32_output=True)
    kv, n = w.Hk - 1, 48
    g = oracle.bwd_group(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], h["dO"], L, w.scale, 0, kv,
                         T - n, T)
    hs = slice(kv * G, (kv + 1) * G)
    tag = f"{name} (kv={kv}, tokens {T - n}..{T - 1})"
    check(f"{tag} dQ", to64(dQ[0, hs, T - n:]), g["dQ"], w.dtype)
    check(f"{tag} dK", to64(dK[0, kv, T - n:]), g["dK"][T - n:], w.dtype)
    check(f"{tag} dV", to64(dV[0, kv, T - n:]), g["dV"][T - n:], w.dtype)
    check(f"{tag} dKd", to64(dKd[0, kv, (T - n) * L:]), g["dKd"], w.dtype)
    check(f"{tag} dVd", to64(dVd[0, kv, (T - n) * L:]), g["dVd"], w.dtype)


@pytest.mark.parametrize("scan", [binding.MODA_SCAN_WAVE, binding.MODA_SCAN_CHUNK,
                                  binding.MODA_SCAN_ALL])
def test_depth_scan_ablation_gives_the_operator(scan):
    """The Table 7 shape (T=1024, G=8, L=64): whatever depth rows each query block scores,
    the mask leaves the operator; compared with the oracle in full."""
    w = PW["table7"]
    x = inputs.make(w, seed=61, device=DEV)
    p = binding.problem_for(x["Q"], x["K"], w.L, w.scale)
    O = torch.empty_like(x["Q"])
    lse = torch.empty(x["Q"].shape[:3], device=DEV)
    binding.moda_fwd_depth_scan(p, scan, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], O, lse)
    torch.cuda.synchronize()
    h = oracle_inputs(x)
    Or, lr = oracle.fwd(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], w.L, w.scale)
    check(f"table7 scan {scan} O", to64(O), Or, w.dtype)
    check(f"table7 scan {scan} lse", to64(lse), lr, w.dtype, fp32_output=True)


@pytest.mark.parametrize("name", ["table2_G2", "table2_T4096", "table7"])
def test_every_key_gradient_under_sparse_upstream(name):
    """dO zero outside a token set S, so the oracle's backward restricted to S is exact for
    every gradient: every dK and dV row of every KV group -- the heavy first key blocks
    included -- is compared, with dQ and the depth gradients of S (the other tokens' depth
    rows and dQ rows must be exactly zero).  G=2 (T=16384, 1024 key-stationary workgroups)
    runs the key pass at two waves per SIMD; T=4096 and the Table 7 shape (256 and 64 key
    blocks) run it split, the heavy blocks' query walks in pieces summed by the reduce."""
    w = PW[name]
    G, T, L = w.G, w.T, w.L
    x = inputs.make(w, seed=62, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = run_fwd(x, w)
    tok = set(range(4)) | set(range(T - 4, T)) | set(np.linspace(0, T - 1, 40).astype(int))
    for c in (1, 3, 5, 37, 64, 127):
        tok |= {c * 128 - 1, c * 128}
    S = np.array(sorted(t for t in tok if 0 <= t < T))
    idx = torch.from_numpy(S).to(DEV)
    dO = torch.zeros_like(x["dO"])
    dO[:, :, idx] = x["dO"][:, :, idx]
    dQ, dK, dV, dKd, dVd = run_bwd(dict(x, dO=dO), w, O, lse)
    torch.cuda.synchronize()
    h = oracle_inputs(dict(x, dO=dO))
    rows = (torch.from_numpy(S)[:, None] * L + torch.arange(L)[None, :]).reshape(-1).to(DEV)
    other = torch.ones(T * L, dtype=torch.bool, device=DEV)
    other[rows] = False
    for kv in range(w.Hk):
        g = oracle.bwd_tokens(h["Q"], h["K"], h["V"], h["Kd"], h["Vd"], h["dO"], L, w.scale, 0,
                              kv, S)
        hs = slice(kv * G, (kv + 1) * G)
        tag = f"{name} sparse dO ({len(S)} tokens) kv={kv}"
        check(f"{tag} dK (all {T} keys)", to64(dK[0, kv]), g["dK"], w.dtype)
        check(f"{tag} dV (all {T} keys)", to64(dV[0, kv]), g["dV"], w.dtype)
        check(f"{tag} dQ", to64(dQ[0, hs][:, idx]), g["dQ"], w.dtype)
        check(f"{tag} dKd", to64(dKd[0, kv, rows]), g["dKd"], w.dtype)
        check(f"{tag} dVd", to64(dVd[0, kv, rows]), g["dVd"], w.dtype)
        assert not torch.any(dKd[0, kv, other] != 0) and not torch.any(dVd[0, kv, other] != 0)
        assert not torch.any(dQ[0, hs][:, ~torch.isin(torch.arange(T, device=DEV), idx)] != 0)
