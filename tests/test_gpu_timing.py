"""GPU: the per-kernel timing hook (moda_timing_arm / _count / _label) brackets
exactly the kernels each entry point launches, in launch order, and stops when
its events run out.  Profiling support only; the outputs themselves are checked
by the parity tests."""
import pytest
import torch

from transformer_attention_moda_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(L):
    w = inputs.Workload("timing", 1, 4, 2, 200, 128, L, chunk=0, dtype="bf16")
    return w, inputs.make(w, seed=11, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))


def test_timing_hook_labels_every_kernel_in_launch_order():
    w, x = _inputs(L=3)
    layers = torch.randn(3, 1, 2, 200, 128, device=DEV).to(torch.bfloat16)
    t = binding.KernelTimer(32)
    try:
        t.arm()
        binding.pack_depth(layers)
        O, lse = binding.fwd(x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], w.L, w.scale)
        binding.bwd(x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], O, lse, x["dO"], w.L, w.scale)
        torch.cuda.synchronize()
        res = t.results()
        t.disarm()
        assert binding.load().moda_timing_count() == 0
    finally:
        t.close()
    labels = [lb for lb, _ in res]
    assert labels == ["pack", "fwd", "bwd_pre", "bwd_depth", "bwd_dq", "bwd_dkdv"], labels
    assert all(ms > 0.0 for _, ms in res), res


def _timed_fwd_bwd_L0(capacity):
    w, x = _inputs(L=0)
    t = binding.KernelTimer(capacity)
    try:
        t.arm()
        O, lse = binding.fwd(x["Q"], x["K"], x["V"], None, None, w.L, w.scale)
        grads = binding.bwd(x["Q"], x["K"], x["V"], None, None, O, lse, x["dO"], w.L, w.scale)
        torch.cuda.synchronize()
        res = t.results()
        t.disarm()
    finally:
        t.close()
    return res, grads


def test_timing_hook_has_no_depth_kernel_at_L0():
    res, _ = _timed_fwd_bwd_L0(32)
    assert [lb for lb, _ in res] == ["fwd", "bwd_pre", "bwd_dq", "bwd_dkdv"], res


def test_timing_hook_stops_when_its_events_run_out():
    res, grads = _timed_fwd_bwd_L0(4)   # two kernels' worth of events
    assert [lb for lb, _ in res] == ["fwd", "bwd_pre"], res
    dQ, dK, dV, dKd, dVd = grads   # the untimed kernels still ran
    assert dKd is None and dVd is None
    for g in (dQ, dK, dV):
        assert bool(torch.isfinite(g.float()).all()) and float(g.float().abs().max()) > 0.0
