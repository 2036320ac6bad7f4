"""moda_bwd_noalloc -- the backward for callers that cannot allocate device memory,
with the library's static per-GPU scratch in place of a workspace -- against the
existing entry point moda_bwd on the same inputs, through the C ABI: two calls in a
row, the second on a smaller problem (the scratch keeps the first call's contents).
The kernels are the same and deterministic, so the gradients must be bitwise equal
(which implies the parity bar)."""
import ctypes

import pytest
import torch

from transformer_attention_moda_amd import binding, inputs
from parity import check, run_fwd, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def compare_once(w, seed):
    x = inputs.make(w, seed=seed, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    O, lse = run_fwd(x, w)
    ref = binding.bwd(x["Q"], x["K"], x["V"], x.get("Kd"), x.get("Vd"), O, lse, x["dO"], w.L,
                      w.scale)
    got = [torch.full_like(r, float("nan")) if r is not None else None for r in ref]
    p = binding.problem_for(x["Q"], x["K"], w.L, w.scale)
    binding.moda_bwd_noalloc(p, x["Q"], x["K"], x["V"], x.get("Kd"), x.get("Vd"), O, lse,
                             x["dO"], *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV", "dKd", "dVd"), got, ref):
        if b is None:
            continue
        print(f"noalloc {w.name} {name}: bitwise equal = {torch.equal(a, b)}", flush=True)
        check(f"noalloc {w.name} {name}", to64(a), to64(b), w.dtype)
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), name


def test_noalloc_backward_matches_workspace_backward_twice_second_smaller():
    big = inputs.Workload("noalloc_big", B=2, Hq=8, Hk=4, T=700, d=128, L=5, chunk=0,
                          dtype="bf16")
    small = inputs.Workload("noalloc_small", B=1, Hq=4, Hk=2, T=130, d=64, L=3, chunk=0,
                            dtype="bf16")
    need_big = binding.moda_bwd_workspace_bytes(binding.problem(2, 8, 4, 700, 128, 5))
    need_small = binding.moda_bwd_workspace_bytes(binding.problem(1, 4, 2, 130, 64, 3))
    assert need_small < need_big <= binding.MODA_NOALLOC_SCRATCH_BYTES
    compare_once(big, 31)
    compare_once(small, 32)


def test_noalloc_backward_fp32_and_no_depth():
    compare_once(inputs.Workload("noalloc_f32", 1, 4, 2, 77, 64, 2, 0, "f32"), 33)
    compare_once(inputs.Workload("noalloc_l0", 1, 4, 2, 200, 128, 0, 0, "bf16"), 34)


def test_noalloc_rejects_problems_beyond_its_scratch():
    # 2 * 16 * 65536 rows at d = 128 with depth rows need about 545 MB of scratch.
    p = binding.problem(2, 16, 8, 65536, 128, 4)
    assert binding.moda_bwd_workspace_bytes(p) > binding.MODA_NOALLOC_SCRATCH_BYTES
    lib = binding.load()
    A = 0x10000
    rc = lib.moda_bwd_noalloc(ctypes.byref(p), *([A] * 13), None)
    assert rc == binding.MODA_ERR_UNSUPPORTED
    assert "scratch" in lib.moda_last_error().decode()
