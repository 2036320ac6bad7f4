"""GPU: libmoda runs on the caller's stream and allocates and synchronises nothing,
so its calls work on a side stream and inside a captured HIP graph.  Results are
compared bitwise with the same calls made eagerly on the default stream (the
kernels are deterministic)."""
import pytest
import torch

from transformer_attention_moda_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _setup(L=4):
    w = inputs.Workload("streams", 1, 4, 2, 300, 128, L, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=23, device=DEV, names=("Q", "K", "V", "Kd", "Vd", "dO"))
    p = binding.problem_for(x["Q"], x["K"], w.L, w.scale)
    out = {
        "O": torch.empty_like(x["Q"]),
        "lse": torch.empty(x["Q"].shape[:3], device=DEV, dtype=torch.float32),
        "dQ": torch.empty_like(x["Q"]), "dK": torch.empty_like(x["K"]),
        "dV": torch.empty_like(x["V"]), "dKd": torch.empty_like(x["Kd"]),
        "dVd": torch.empty_like(x["Vd"]),
        "ws": torch.empty(binding.moda_bwd_workspace_bytes(p), device=DEV, dtype=torch.uint8),
    }
    return p, x, out


def _run(p, x, o):
    binding.moda_fwd(p, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], o["O"], o["lse"])
    binding.moda_bwd(p, x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], o["O"], o["lse"], x["dO"],
                     o["dQ"], o["dK"], o["dV"], o["dKd"], o["dVd"], o["ws"])


NAMES = ("O", "lse", "dQ", "dK", "dV", "dKd", "dVd")


def test_calls_run_on_the_callers_side_stream():
    p, x, o = _setup()
    _run(p, x, o)
    torch.cuda.synchronize()
    ref = {k: o[k].clone() for k in NAMES}
    for k in NAMES:
        o[k].zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run(p, x, o)
    s.synchronize()
    for k in NAMES:
        assert torch.equal(o[k], ref[k]), k


def test_graph_capture_replays_match_eager():
    p, x, o = _setup()
    _run(p, x, o)
    torch.cuda.synchronize()
    ref = {k: o[k].clone() for k in NAMES}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(p, x, o)
    torch.cuda.synchronize()
    a = torch.randn(256, 256, device=DEV)
    for rep in range(3):
        for k in NAMES:   # eager work between replays
            o[k].zero_()
        b = (a @ a).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in NAMES:
            assert torch.equal(o[k], ref[k]), (rep, k)
        assert torch.isfinite(b)
