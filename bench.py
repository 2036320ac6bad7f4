#!/usr/bin/env python3
"""MoDA operator benchmark on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: pack the layer-major depth K and V into the
token-major layout, run the forward (O and log-sum-exp), then the backward
(dQ, dK, dV, dK_depth, dV_depth).  The default workload is the 64K-token long
sequence (B=1, Hq=16, Hk=8, T=65536, d=128, L=24, bf16).

Printed: one JSON line.  `value` is algorithmic forward+backward TFLOP/s of
the whole step (forward FLOP = 4 d B Hq (T(T+1)/2 + T L), backward = 2.5x
forward); the same step with L=0 (no depth: plain causal attention through
the same entry points) gives the overhead of the depth path.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E (published)


def fwd_flops(w, L=None):
    L = w.L if L is None else L
    pairs = w.T * (w.T + 1) // 2 + w.T * L
    return 4.0 * w.d * w.B * w.Hq * pairs


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_64k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-l0", action="store_true", help="skip the L=0 comparison run")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (a "
                         "kernel of known traffic for scaling hardware byte counters)")
    return ap.parse_args()


class Step:
    """Buffers and the launches of one step, with per-entry-point events."""

    def __init__(self, w, L, seed=0):
        import torch
        from transformer_attention_moda_amd import binding, inputs
        self.torch, self.mb, self.w, self.L = torch, binding, w, L
        dev = "cuda:0"
        names = ["Q", "K", "V", "dO"] + (["layers_K", "layers_V"] if L > 0 else [])
        x = inputs.make(w.with_(L=L), seed=seed, device=dev, names=names)
        self.x = x
        self.p = binding.problem_for(x["Q"], x["K"], L, w.scale, chunk=0)
        B, Hk, T, d = w.B, w.Hk, w.T, w.d
        empty = lambda shape: torch.empty(shape, device=dev, dtype=torch.bfloat16)  # noqa: E731
        self.Kd = empty((B, Hk, T * L, d)) if L > 0 else None
        self.Vd = empty((B, Hk, T * L, d)) if L > 0 else None
        self.O = torch.empty_like(x["Q"])
        self.lse = torch.empty((w.B, w.Hq, T), device=dev, dtype=torch.float32)
        self.dQ, self.dK, self.dV = (torch.empty_like(x["Q"]), torch.empty_like(x["K"]),
                                     torch.empty_like(x["V"]))
        self.dKd = torch.empty_like(self.Kd) if L > 0 else None
        self.dVd = torch.empty_like(self.Vd) if L > 0 else None
        nws = binding.moda_bwd_workspace_bytes(self.p)
        self.ws = torch.empty(max(nws, 256), device=dev, dtype=torch.uint8)
        if L > 0:
            self.pp = binding.problem(B, Hk, Hk, T, d, L, 1.0, binding.MODA_BF16)
        self.events = []

    def run(self):
        mb, x = self.mb, self.x
        if self.L > 0:
            mb.moda_pack_depth(self.pp, x["layers_K"], self.Kd)
            mb.moda_pack_depth(self.pp, x["layers_V"], self.Vd)
        mb.moda_fwd(self.p, x["Q"], x["K"], x["V"], self.Kd, self.Vd, self.O, self.lse)
        mb.moda_bwd(self.p, x["Q"], x["K"], x["V"], self.Kd, self.Vd, self.O, self.lse, x["dO"],
                    self.dQ, self.dK, self.dV, self.dKd, self.dVd, self.ws)

    def timed(self, steps, warmup):
        """Average step time (ms) over `steps`, and per kernel the average
        duration (ms) and launches per step, from HIP events libmoda records
        around each of its kernels on the stream they run on."""
        torch = self.torch
        for _ in range(warmup):
            self.run()
        torch.cuda.synchronize()
        timer = self.mb.KernelTimer(capacity=16 * 2 * steps + 16)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        timer.arm()
        wall0 = time.perf_counter()
        t0.record()
        for _ in range(steps):
            self.run()
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        results = timer.results()
        timer.disarm()
        kernels = {}
        for label, ms in results:
            k = kernels.setdefault(label, {"total_ms": 0.0, "launches": 0})
            k["total_ms"] += ms
            k["launches"] += 1
        timer.close()
        for k in kernels.values():
            k["avg_ms"] = k["total_ms"] / k["launches"]
            k["per_step"] = k["launches"] / steps
        return t0.elapsed_time(t1) / steps, kernels, wall


def traffic_for(label):
    """Per-launch HBM traffic of a kernel from the committed rocprofv3 counter
    summary (profiles/traffic.txt: FETCH_SIZE and WRITE_SIZE, each scaled by
    the factor a plain copy of known size gives), or None when the kernel's
    sources changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
        if f.get("kernel") != label:
            continue
        h = hashlib.sha256()
        for src in f.get("sources", "").split(","):
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest()[:16] != f.get("sha"):
            return None
        return {"fetch_bytes": float(f["fetch_bytes"]), "write_bytes": float(f["write_bytes"]),
                "bytes": float(f["fetch_bytes"]) + float(f["write_bytes"])}
    return None


def fwd_overhead(step, step0, rounds=8):
    """Depth overhead of the forward measured with interleaved launches: each round
    times moda_fwd with depth (L) and without (L=0) back to back, so clock drift
    affects both alike.  Returns median milliseconds of each."""
    torch, mb = step.torch, step.mb
    x, x0 = step.x, step0.x
    tl, t0 = [], []
    for _ in range(rounds):
        for st, xx, acc in ((step, x, tl), (step0, x0, t0)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(2):
                mb.moda_fwd(st.p, xx["Q"], xx["K"], xx["V"], st.Kd, st.Vd, st.O, st.lse)
            e1.record()
            torch.cuda.synchronize()
            acc.append(e0.elapsed_time(e1) / 2)
    tl.sort()
    t0.sort()
    return tl[len(tl) // 2], t0[len(t0) // 2]


def kernel_work(label, w):
    """Algorithmic work of one launch of a libmoda kernel: (bound, amount, unit).

    Sequence pairs P_s = B Hq T(T+1)/2 and depth pairs P_d = B Hq T L are the
    visible (query, key) pairs.  FLOP counts are 2 d per pair and product:
    forward = S and O products over all pairs (4 d); backward = 5 products
    (S recomputed, dP, dV, dK, dQ), of which bwd_dkdv does the four sequence
    ones besides dQ, bwd_depth all five depth ones, bwd_dq the sequence dQ
    product (its own S and dP are recomputation).  Memory-bound kernels count
    the bytes they must move once (bwd_depth: the depth K/V read, their
    gradients written, the query rows' Q and dO read, and the fp32 depth part
    of dQ written for bwd_dq)."""
    d, B, Hq, Hk, T, L = w.d, w.B, w.Hq, w.Hk, w.T, w.L
    Ps, Pd = B * Hq * T * (T + 1) / 2, B * Hq * T * L
    q_bytes, dep_bytes, rows = B * Hq * T * d * 2, B * Hk * T * L * d * 2, B * Hq * T
    if label == "fwd":
        return "mfma", 4 * d * (Ps + Pd), "FLOP"
    if label == "bwd_dkdv":
        return "mfma", 8 * d * Ps, "FLOP"
    if label == "bwd_dq":
        return "mfma", 2 * d * Ps, "FLOP"
    if label == "bwd_depth":
        return "hbm", 4 * dep_bytes + 2 * q_bytes + 8 * rows + (4 * d * rows if L > 0 else 0), "B"
    if label == "bwd_pre":
        return "hbm", 2 * q_bytes + 12 * rows, "B"
    if label == "pack":
        return "hbm", 2 * dep_bytes, "B"   # one of K or V per launch: read + write
    return None, 0, None


def cpu_baseline(w, step, seconds):
    """Time the CPU oracle on a bounded sample of the same workload: the full
    forward+backward of the last n tokens of one KV group (G query heads)."""
    import numpy as np
    import oracle
    from transformer_attention_moda_amd import inputs as inp
    x = step.x
    G, T, L, d = w.G, w.T, w.L, w.d
    th = oracle.num_threads()

    def sample(n):
        t_lo = T - n
        sub = {
            "Q": inp.to_host_storage(x["Q"][:1, :G]),
            "dO": inp.to_host_storage(x["dO"][:1, :G]),
            "K": inp.to_host_storage(x["K"][:1, :1]),
            "V": inp.to_host_storage(x["V"][:1, :1]),
        }
        for name, src in (("Kd", step.Kd), ("Vd", step.Vd)):
            full = np.zeros((1, 1, T * L, d), np.uint16)
            full[0, 0, t_lo * L:] = inp.to_host_storage(src[0, 0, t_lo * L:])
            sub[name] = full
        t0 = time.perf_counter()
        oracle.bwd_group(sub["Q"], sub["K"], sub["V"], sub["Kd"], sub["Vd"], sub["dO"], L,
                         w.scale, 0, 0, t_lo, T)
        dt = time.perf_counter() - t0
        pairs = sum(t + 1 + L for t in range(t_lo, T)) * G
        return dt, 3.5 * 4.0 * d * pairs, t_lo

    sample(1)                      # start the OpenMP pool
    n = 8
    dt, fl, _ = sample(n)
    while dt < seconds / 8 and n < T:   # grow the sample until it takes a measurable time
        n = min(T, n * 4)
        dt, fl, _ = sample(n)
    n = int(max(n, min(T, n * seconds / max(dt, 1e-3))))
    dt, fl, t_lo = sample(n)
    return {
        "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": th, "kind": "oracle",
        "sample": (f"fp64 forward+backward of tokens {t_lo}..{T - 1} of one KV group "
                   f"({G} query heads, b=0, kv=0) of the {w.name} workload; "
                   f"{dt:.1f} s on {th} threads; algorithmic FLOP of the sample "
                   f"(3.5 x 4 d x visible pairs) / wall time"),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from transformer_attention_moda_amd import binding, inputs
    binding.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = inputs.WORKLOADS[args.workload]
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, device="cuda:0", dtype=torch.uint8).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step = Step(w, w.L, seed=0)
    ms, kernels, wall = step.timed(args.steps, args.warmup)
    f_fwd, f_all = fwd_flops(w), 3.5 * fwd_flops(w)
    value = f_all / (ms * 1e-3) / 1e12

    res0 = None
    if not args.no_l0:
        del step.x["layers_K"], step.x["layers_V"]
        torch.cuda.empty_cache()
        s0 = Step(w, 0, seed=0)
        ms0, k0, _ = s0.timed(args.steps, args.warmup)
        fl, f0 = fwd_overhead(step, s0)
        res0 = {"ms_per_step": ms0, "kernels": k0, "fwd_interleaved": (fl, f0)}
        del s0
        torch.cuda.empty_cache()

    def roof(label, k, wl):
        bound, amount, _ = kernel_work(label, wl)
        if bound == "mfma":
            ach, peak, unit = amount / (k["avg_ms"] * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = amount / (k["avg_ms"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4)}

    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["per_step"])
    roofline = dict(roof(dom, kernels[dom], w), traffic=traffic_for(dom), kernel=dom,
                    avg_ms=round(kernels[dom]["avg_ms"], 4))
    per_kernel = {n: dict(roof(n, k, w), avg_ms=round(k["avg_ms"], 4),
                          launches_per_step=k["per_step"]) for n, k in kernels.items()}

    cpu = None
    if not args.no_cpu_baseline:
        if step.Kd is None:
            step = Step(w, w.L, seed=0)
            step.run()
            torch.cuda.synchronize()
        cpu = cpu_baseline(w, step, args.cpu_seconds)

    out = {
        "metric": "MoDA fwd+bwd TFLOP/s bf16 at T=64K (% MFMA peak); overhead vs own L=0 path",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "T": w.T, "d": w.d,
                   "L": w.L, "step": "pack depth K,V + forward + backward",
                   "chunk_tokens": binding.moda_fwd_chunk_tokens(step.p)},
        "pct_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "roofline": roofline,
        "fwd": {"ms": round(kernels["fwd"]["avg_ms"], 3),
                "tflops": round(f_fwd / (kernels["fwd"]["avg_ms"] * 1e-3) / 1e12, 2),
                "frac": round(f_fwd / (kernels["fwd"]["avg_ms"] * 1e-3) / 1e12 /
                              MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels": per_kernel,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    if res0:
        k0 = res0["kernels"]
        fwd_l, fwd_0 = kernels["fwd"]["avg_ms"], k0["fwd"]["avg_ms"]
        bwd_l = sum(v["avg_ms"] * v["per_step"] for n, v in kernels.items() if n.startswith("bwd"))
        bwd_0 = sum(v["avg_ms"] * v["per_step"] for n, v in k0.items() if n.startswith("bwd"))
        out["l0"] = {"ms_per_step": round(res0["ms_per_step"], 3), "fwd_ms": round(fwd_0, 3),
                     "bwd_ms": round(bwd_0, 3),
                     "fwd_tflops": round(fwd_flops(w, 0) / (fwd_0 * 1e-3) / 1e12, 2)}
        fl, f0 = res0["fwd_interleaved"]
        out["l0"]["fwd_interleaved_ms"] = {"L": round(fl, 3), "L0": round(f0, 3)}
        out["overhead"] = {
            "fwd_interleaved": round((fl - f0) / f0, 4),
            "fwd": round((fwd_l - fwd_0) / fwd_0, 4),
            "fwd_bwd": round((fwd_l + bwd_l - fwd_0 - bwd_0) / (fwd_0 + bwd_0), 4),
            "step": round((ms - res0["ms_per_step"]) / res0["ms_per_step"], 4),
            "fwd_pages_convention": round((fwd_l - fwd_0) / fwd_l, 4),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
