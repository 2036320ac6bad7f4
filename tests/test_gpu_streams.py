"""GPU: libmoda runs on the caller's stream and allocates and synchronises nothing,
so its calls work on a side stream and inside a captured HIP graph.  (On small problems
the backward's key pass runs on a second stream of the library's, forked from the
caller's stream by an event and joined back into it by another: work the caller enqueues
after the call still sees every gradient.)  Results are compared bitwise with the same
calls made eagerly on the default stream (the kernels are deterministic)."""
import pytest
import torch

from transformer_attention_moda_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# (B, Hq, Hk, T, d): one shape whose backward runs the key pass whole, and one small enough
# (8 key blocks of one KV head) that it splits the walks and adds the pieces in a second kernel.
SHAPES = [(1, 4, 2, 300, 128), (1, 8, 1, 1024, 64)]


def _setup(L=4, shape=SHAPES[0]):
    w = inputs.Workload("streams", *shape, L, chunk=0, dtype="bf16")
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


@pytest.mark.parametrize("shape", SHAPES)
def test_calls_run_on_the_callers_side_stream(shape):
    p, x, o = _setup(shape=shape)
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


@pytest.mark.parametrize("shape", SHAPES)
def test_work_enqueued_after_the_backward_sees_its_gradients(shape):
    """The key pass's dK and dV, written on the library's second stream, are complete for a
    copy the caller enqueues on its own stream right after the call, with no synchronisation
    between them."""
    p, x, o = _setup(shape=shape)
    _run(p, x, o)
    torch.cuda.synchronize()
    ref = {k: o[k].clone() for k in NAMES}
    s = torch.cuda.Stream()
    for rep in range(3):
        for k in NAMES:
            o[k].fill_(float("nan"))
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            _run(p, x, o)
            copies = {k: o[k].clone() for k in NAMES}
        s.synchronize()
        for k in NAMES:
            assert torch.equal(copies[k], ref[k]), (rep, k)


@pytest.mark.parametrize("shape", SHAPES)
def test_graph_capture_replays_match_eager(shape):
    p, x, o = _setup(shape=shape)
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


def test_append_and_decode_step_in_a_captured_graph():
    """A serving step as a graph: append one layer's entries for the last 4 tokens into a
    slot of the packed depth cache, then decode the last token; three replays with eager
    work between them match the eager step bitwise."""
    w = inputs.Workload("decode_graph", 1, 8, 2, 300, 128, 4, chunk=0, dtype="bf16")
    x = inputs.make(w, seed=29, device=DEV, names=("Q", "K", "V", "Kd", "Vd"))
    p = binding.problem_for(x["Q"], x["K"], w.L, w.scale)
    layer = inputs.normal((1, w.Hk, 4, w.d), seed=29, tensor="layers_K", device=DEV)
    q = x["Q"][:, :, -1].contiguous()
    packed = x["Kd"].clone()
    O = torch.empty_like(q)
    lse = torch.empty((1, w.Hq), device=DEV, dtype=torch.float32)
    ws = torch.empty(binding.moda_decode_workspace_bytes(p), device=DEV, dtype=torch.uint8)

    def step():
        binding.moda_depth_append(p, layer, 2, w.T - 4, packed)
        binding.moda_decode(p, w.T - 1, q, x["K"], x["V"], packed, x["Vd"], O, lse, ws)

    step()
    torch.cuda.synchronize()
    ref = (packed.clone(), O.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    a = torch.randn(256, 256, device=DEV)
    for rep in range(3):
        packed.copy_(x["Kd"])
        O.zero_()
        lse.zero_()
        b = (a @ a).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(packed, ref[0]) and torch.equal(O, ref[1]) and torch.equal(lse, ref[2]), rep
        assert torch.isfinite(b)
