"""Helpers shared by the GPU parity tests: tolerance checks and oracle calls."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from transformer_attention_moda_amd import binding, inputs

# Tolerances of the parity bar: max |x - ref| and ||x - ref||_F / ||ref||_F.
TOL = {"bf16": (2e-2, 1e-2), "f32": (2e-2, 1e-4)}


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    nr = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nr) if nr > 0 else float(np.linalg.norm(diff))
    return mx, rel


# Edge shapes outside the five workloads (up to 32 query heads per KV head, up to
# 1024 depth slots) have bf16 outputs that are large, or small sums of many large
# terms.  The bf16 path rounds each weight P (and each dS) to bfloat16 before its
# MFMA, and rounds every output once more (round-to-nearest-even, unit roundoff
# u = 2^-8 for an 8-bit significand).  To first order, a sum of terms a_i b_i whose
# a_i are so rounded is off by at most u * sum |a_i b_i|, and the output rounding by
# u |x|.  So for edge shapes the element bound of a bf16-stored output is
#   2e-2 + 2^-8 (|ref| + A),
# A being the sum of the absolute values of that output's terms (oracle.brute.abs_terms);
# fp32 outputs (the log-sum-exp, and everything of the fp32 path) keep the plain 2e-2.
# The relative Frobenius bound is never widened.  The five workloads use the plain
# bound for every output.
BF16_ROUNDING = 2.0 ** -8

# Every check appends (name, fraction of the element bound used, fraction of the
# relative bound used); tests/conftest.py writes them out when MODA_PARITY_REPORT
# names a file.
MARGINS = []


def check(name, got, ref, dtype, report=None, edge=False, fp32_output=False, terms=None):
    """Assert the parity bar for one output tensor.  edge: allow the bf16 rounding terms
    (bf16-stored outputs only), with `terms` the absolute-term sums A of the output;
    fp32_output: the tensor is stored in fp32 (lse), so no rounding term applies."""
    mx_tol, rel_tol = TOL[dtype]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mx, rel = errors(got, ref)
    rounding = BF16_ROUNDING if (edge and dtype == "bf16" and not fp32_output) else 0.0
    A = 0.0 if terms is None else np.asarray(terms, np.float64)
    bound = mx_tol + rounding * (np.abs(ref) + A)
    used = float((np.abs(got - ref) / bound).max()) if ref.size else 0.0
    ok = np.isfinite(mx) and used <= 1.0 and rel <= rel_tol
    term = f"{mx_tol:g} + 2^-8(|ref| + A)" if rounding else f"{mx_tol:g}"
    line = (f"{name}: max_abs={mx:.3e} (<= {term}; {100 * used:.1f}% of the element bound) "
            f"rel_fro={rel:.3e} (<= {rel_tol:g}; {100 * rel / rel_tol:.1f}%)")
    print(line, flush=True)
    MARGINS.append((name, used, rel / rel_tol))
    if report is not None:
        report.append(line)
    assert ok, line


def host(t):
    return inputs.to_host_storage(t)


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_fwd(x, w, chunk=0, causal=True, window=0):
    return binding.fwd(x["Q"], x["K"], x["V"], x.get("Kd"), x.get("Vd"), w.L, w.scale,
                       chunk=chunk, causal=causal, window=window)


def run_bwd(x, w, O, lse, chunk=0, causal=True, window=0):
    return binding.bwd(x["Q"], x["K"], x["V"], x.get("Kd"), x.get("Vd"), O, lse, x["dO"], w.L,
                       w.scale, chunk=chunk, causal=causal, window=window)


def oracle_inputs(x):
    return {k: (host(v) if v is not None else None) for k, v in x.items()}


def rows_array(B, Hq, tokens, heads=None):
    heads = range(Hq) if heads is None else heads
    return np.array([[b, h, t] for b in range(B) for h in heads for t in tokens], np.int64)


def gather_rows(t, rows):
    """t[b, h, t, ...] at each (b, h, t) of rows, on the host in float64."""
    idx = torch.from_numpy(rows).to(t.device)
    return to64(t[idx[:, 0], idx[:, 1], idx[:, 2]])
