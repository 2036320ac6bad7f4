"""moda_attention: the operator as one differentiable torch call.  Its output is moda_fwd's
and the gradients torch autograd returns through it are moda_bwd's, bitwise (moda_fwd and
moda_bwd are compared with the oracle in test_gpu_parity.py), for bf16 and fp32 storage,
with and without depth rows, causal and non-causal, with a depth window."""
import pytest
import torch

from transformer_attention_moda_amd import binding as mb
from transformer_attention_moda_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [("bf16", 3, True, 0), ("bf16", 0, True, 0), ("bf16", 5, False, 2), ("bf16", 4, True, 1),
         ("f32", 3, True, 0)]


@pytest.mark.parametrize("dtype,L,causal,window", CASES)
def test_autograd_gives_the_explicit_backward(dtype, L, causal, window):
    w = inputs.Workload("autograd", 1, 4, 2, 130, 64, L, 0, dtype)
    print(f"case moda_attention {dtype} L={L} causal={causal} window={window}", flush=True)
    x = inputs.make(w, seed=11, device="cuda:0", names=("Q", "K", "V", "Kd", "Vd", "dO"))
    names = ("Q", "K", "V") + (("Kd", "Vd") if L else ())
    leaf = {n: x[n].clone().requires_grad_(True) for n in names}
    O = mb.moda_attention(leaf["Q"], leaf["K"], leaf["V"], leaf.get("Kd"), leaf.get("Vd"), L,
                          scale=w.scale, causal=causal, window=window)
    O.backward(x["dO"])
    O_ref, lse_ref = mb.fwd(x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], L, w.scale,
                            causal=causal, window=window)
    grads = mb.bwd(x["Q"], x["K"], x["V"], x["Kd"], x["Vd"], O_ref, lse_ref, x["dO"], L, w.scale,
                   causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(O.detach(), O_ref)
    for n, g in zip(("Q", "K", "V", "Kd", "Vd"), grads):
        if n in leaf:
            assert leaf[n].grad is not None and torch.equal(leaf[n].grad, g), n
