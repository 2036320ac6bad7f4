"""Seeded synthetic inputs for the MoDA operator.

This module holds workload shapes and random-number generation only; none of
the operator's arithmetic lives here.  Both the HIP library's callers and the
CPU oracle's callers take their inputs from it.

The pages measure the kernel on synthetic shapes with no dataset (the
"Kernel Efficiency" tables of the MoDA README; the kernel ablation of the
paper summary), so every workload here is synthetic: Q, K, V, K_depth,
V_depth and the upstream gradient dO are i.i.d. standard normal, drawn in
fp32 from a seeded torch generator and rounded once to bfloat16
(round-to-nearest-even) for bf16 workloads.  Depth rows are token-major:
row t*L + l is token t's slot l.  One workload scales K_depth by 0.5 (exact in
bfloat16) so that depth and sequence scores compete.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hk: int
    T: int
    d: int
    L: int
    chunk: int          # tokens per query chunk requested (a tiling hint)
    dtype: str          # "bf16" or "f32"
    kd_scale: float = 1.0
    bwd: bool = False   # whether the workload's parity covers the gradients

    @property
    def G(self) -> int:
        return self.Hq // self.Hk

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32: the value passed across the C ABI."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_fp32", B=1, Hq=4, Hk=2, T=128, d=64, L=4, chunk=16, dtype="f32"),
        Workload("small_model", B=2, Hq=16, Hk=8, T=2048, d=64, L=16, chunk=64, dtype="bf16",
                 kd_scale=0.5),
        Workload("layer_1p5b_8k", B=1, Hq=16, Hk=4, T=8192, d=128, L=32, chunk=64,
                 dtype="bf16"),
        Workload("long_64k", B=1, Hq=16, Hk=8, T=65536, d=128, L=24, chunk=128, dtype="bf16"),
        Workload("train_4k", B=4, Hq=16, Hk=8, T=4096, d=128, L=32, chunk=64, dtype="bf16",
                 bwd=True),
    )
}

# The kernel workloads of the pages' efficiency tables (README "Kernel Efficiency",
# bf16, forward and backward, B=1, d=64, Hk=8): the sequence-length sweep (G=8, L=64),
# the GQA-group sweep (T=16384, L=64, Hq=8G) and the depth sweep (T=16384, G=8), and
# the kernel-ablation shape of the paper summary's experiments (Table 7: T=1024, G=8,
# L=64).  The pages' chunk C=64 is their kernel's tiling; these run with this
# library's default tiling (chunk 0).
PAGE_WORKLOADS = {
    w.name: w
    for w in (
        [Workload(f"table2_T{T}", B=1, Hq=64, Hk=8, T=T, d=64, L=64, chunk=0, dtype="bf16",
                  bwd=True) for T in (4096, 8192, 16384, 32768, 65536)]
        + [Workload(f"table2_G{G}", B=1, Hq=8 * G, Hk=8, T=16384, d=64, L=64, chunk=0,
                    dtype="bf16", bwd=True) for G in (2, 4, 16, 32)]
        + [Workload(f"table2_L{L}", B=1, Hq=64, Hk=8, T=16384, d=64, L=L, chunk=0, dtype="bf16",
                    bwd=True) for L in (128, 256)]
        + [Workload("table7", B=1, Hq=64, Hk=8, T=1024, d=64, L=64, chunk=0, dtype="bf16",
                    bwd=True)]
    )
}
# table2_T16384 is also the G = 8 point of the group sweep and the L = 64 point of the
# depth sweep.

TENSOR_IDS = {"Q": 0, "K": 1, "V": 2, "Kd": 3, "Vd": 4, "dO": 5, "layers_K": 6, "layers_V": 7}


def shapes(w: Workload) -> dict:
    return {
        "Q": (w.B, w.Hq, w.T, w.d), "K": (w.B, w.Hk, w.T, w.d), "V": (w.B, w.Hk, w.T, w.d),
        "Kd": (w.B, w.Hk, w.T * w.L, w.d), "Vd": (w.B, w.Hk, w.T * w.L, w.d),
        "dO": (w.B, w.Hq, w.T, w.d),
        "layers_K": (w.L, w.B, w.Hk, w.T, w.d), "layers_V": (w.L, w.B, w.Hk, w.T, w.d),
    }


def normal(shape, seed: int, tensor: str, device="cpu", dtype=torch.bfloat16,
           scale: float = 1.0) -> torch.Tensor:
    """Seeded N(0,1) draw in fp32, times `scale`, rounded once to `dtype`."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) * 64 + TENSOR_IDS[tensor])
    x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def make(w: Workload, seed: int = 0, device="cpu", names=("Q", "K", "V", "Kd", "Vd"),
         depth_layout: str = "packed") -> dict:
    """Inputs of workload `w` as torch tensors on `device`.

    depth_layout "packed" gives K_depth/V_depth as [B,Hk,T*L,d]; "layers" also
    draws the layer-major [L,B,Hk,T,d] tensors named layers_K / layers_V."""
    sh = shapes(w)
    out = {}
    for n in names:
        if n in ("Kd", "Vd") and w.L == 0:
            out[n] = None
            continue
        sc = w.kd_scale if n in ("Kd", "layers_K") else 1.0
        out[n] = normal(sh[n], seed, n, device, w.torch_dtype, sc)
    return out


def to_host_storage(t: torch.Tensor) -> np.ndarray:
    """Exact host copy for the oracle: bf16 -> uint16 bit patterns, fp32/fp64 as is."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
