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
the same entry points) gives the overhead of the depth path.  `aux` adds the
1.5B-like layer's forward overhead against its L=0 path, cold-cache HBM rates of
the small-model forward and the training-shape forward+backward, and the depth
utilisation of the tiling.

`--suite pages` prints one JSON line per kernel workload of the pages' efficiency
tables (sequence, group and depth sweeps at d=64) and per depth-scan ablation
mode; `--suite decode` one line each for the decoding step, the depth-cache
append and the non-causal and windowed variants at the 64K shape; `--suite
ceiling` one line per setting of the matrix-core rate probe (libmoda_probe.so):
the chip's sustained bf16 MFMA rate and clock with no memory traffic, the
context for the attention kernels' fractions of the nominal peak.
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
    ap.add_argument("--workload", default="long_64k",
                    help="a workload of inputs.WORKLOADS or inputs.PAGE_WORKLOADS (default: the 64K one)")
    ap.add_argument("--suite", choices=["pages", "decode", "ablation", "ceiling"], default=None,
                    help="print one JSON line per workload of a measurement suite instead")
    ap.add_argument("--no-aux", action="store_true", help="skip the auxiliary measurements")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-l0", action="store_true", help="skip the L=0 comparison run")
    ap.add_argument("--no-same-cache", action="store_true",
                    help="decode suite: skip the back-to-back calls on one cache (so that a "
                         "kernel trace holds only calls that cycle through the caches)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain copy of this many MiB first through the packer with "
                         "L=1 (a kernel of known traffic for scaling hardware byte counters)")
    return ap.parse_args()


class Step:
    """Buffers and the launches of one step, with per-entry-point events.  pack: the
    step starts by packing layer-major depth K and V (else the packed depth rows are
    drawn directly); bwd: the step includes the backward."""

    def __init__(self, w, L, seed=0, pack=True, bwd=True, causal=True, window=0):
        import torch
        from transformer_attention_moda_amd import binding, inputs
        self.torch, self.mb, self.w, self.L = torch, binding, w, L
        self.pack, self.bwd = pack and L > 0, bwd
        dev = "cuda:0"
        names = ["Q", "K", "V"] + (["dO"] if bwd else [])
        if L > 0:
            names += ["layers_K", "layers_V"] if self.pack else ["Kd", "Vd"]
        x = inputs.make(w.with_(L=L), seed=seed, device=dev, names=names)
        self.x = x
        self.p = binding.problem_for(x["Q"], x["K"], L, w.scale, chunk=0, causal=causal,
                                     window=window)
        B, Hk, T, d = w.B, w.Hk, w.T, w.d
        empty = lambda shape: torch.empty(shape, device=dev, dtype=torch.bfloat16)  # noqa: E731
        if self.pack:
            self.Kd = empty((B, Hk, T * L, d))
            self.Vd = empty((B, Hk, T * L, d))
        else:
            self.Kd, self.Vd = x.get("Kd"), x.get("Vd")
        self.O = torch.empty_like(x["Q"])
        self.lse = torch.empty((w.B, w.Hq, T), device=dev, dtype=torch.float32)
        if bwd:
            self.dQ, self.dK, self.dV = (torch.empty_like(x["Q"]), torch.empty_like(x["K"]),
                                         torch.empty_like(x["V"]))
            self.dKd = torch.empty_like(self.Kd) if L > 0 else None
            self.dVd = torch.empty_like(self.Vd) if L > 0 else None
            nws = binding.moda_bwd_workspace_bytes(self.p)
            self.ws = torch.empty(max(nws, 256), device=dev, dtype=torch.uint8)
        if self.pack:
            self.pp = binding.problem(B, Hk, Hk, T, d, L, 1.0, binding.MODA_BF16)
        self.events = []

    def run(self):
        mb, x = self.mb, self.x
        if self.pack:
            mb.moda_pack_depth(self.pp, x["layers_K"], self.Kd)
            mb.moda_pack_depth(self.pp, x["layers_V"], self.Vd)
        mb.moda_fwd(self.p, x["Q"], x["K"], x["V"], self.Kd, self.Vd, self.O, self.lse)
        if self.bwd:
            mb.moda_bwd(self.p, x["Q"], x["K"], x["V"], self.Kd, self.Vd, self.O, self.lse,
                        x["dO"], self.dQ, self.dK, self.dV, self.dKd, self.dVd, self.ws)

    def free(self):
        for k in list(vars(self)):
            if k not in ("torch", "mb", "w", "L", "p"):
                delattr(self, k)
        self.torch.cuda.empty_cache()

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


def traffic_for(label, workload):
    """Per-launch HBM traffic of a kernel at a workload from the committed rocprofv3
    counter summary (profiles/traffic.txt: FETCH_SIZE and WRITE_SIZE, each scaled by
    the factor a plain copy of known size gives), or None when that workload was not
    profiled or the kernel's sources changed since its counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
        if f.get("kernel") != label or f.get("workload") != workload:
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
        "cpu_model": cpu_model(),
        "sample": (f"fp64 forward+backward of tokens {t_lo}..{T - 1} of one KV group "
                   f"({G} query heads, b=0, kv=0) of the {w.name} workload; "
                   f"{dt:.1f} s on {th} threads; algorithmic FLOP of the sample "
                   f"(3.5 x 4 d x visible pairs) / wall time"),
    }


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def depth_eta(w, scan=0, window=0, rows_per_wg=None):
    """Depth utilisation of the forward's tiling: the fraction of the depth scores it
    computes that the mask keeps (the "Depth Utilization" of the pages' efficiency tables).
    Each 32-row query block (one wave) scores 32x32 MFMA blocks of depth rows: of its own
    tokens (scan 0), of its workgroup chunk's (1), or all of the KV head's (2); every
    query sees exactly W of them.  rows_per_wg: the library's tiling for w by default."""
    G, T, L = w.G, w.T, w.L
    if rows_per_wg is None:
        from transformer_attention_moda_amd import binding as mb
        rows_per_wg = G * mb.moda_fwd_chunk_tokens(
            mb.problem(w.B, w.Hq, w.Hk, w.T, w.d, w.L, w.scale, chunk=w.chunk))
    W = window if window else L
    if L == 0:
        return None
    TG = T * G
    computed = 0
    for c in range((TG + rows_per_wg - 1) // rows_per_wg):
        r0 = c * rows_per_wg
        for wv in range(rows_per_wg // 32):
            fw = r0 + 32 * wv
            if scan == 0:
                first, last = min(fw // G, T - 1), min((fw + 31) // G, T - 1)
            elif scan == 1:
                first, last = min(r0 // G, T - 1), min((r0 + rows_per_wg - 1) // G, T - 1)
            else:
                first, last = 0, T - 1
            computed += -(-((last - first + 1) * W) // 32) * 32 * 32
    return w.Hq * T * W / (w.Hk * computed)


def fwd_bytes(w, L=None, W=None):
    """Bytes the forward must move once: Q read, O written, K, V and the visible depth
    rows read, lse written."""
    L = w.L if L is None else L
    W = L if W is None else W
    eb = 2
    return (eb * (2 * w.B * w.Hq * w.T * w.d + 2 * w.B * w.Hk * w.T * w.d
                  + 2 * w.B * w.Hk * w.T * W * w.d) + 4 * w.B * w.Hq * w.T)


def bwd_bytes(w):
    """Bytes the backward must move once: Q, O, dO read and dQ written; K, V read and dK,
    dV written; the depth rows read and their gradients written; lse read."""
    eb = 2
    return (eb * (4 * w.B * w.Hq * w.T * w.d + 4 * w.B * w.Hk * w.T * w.d
                  + 4 * w.B * w.Hk * w.T * w.L * w.d) + 4 * w.B * w.Hq * w.T)


def events_ms(torch, fn, reps, flush=None):
    """Median milliseconds of fn() over reps runs, timed with events on the current
    stream; flush() (untimed) runs before each."""
    out = []
    for _ in range(reps):
        if flush:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    out.sort()
    return out[len(out) // 2]


def cold_rates(torch, inputs):
    """HBM rate with cold caches: before each timed run a 1 GiB buffer is written, which
    evicts the 256 MB last-level cache and the L2s.  The small-model forward and the
    training-shape forward+backward, each against the bytes it must move once."""
    flush_buf = torch.empty(1 << 30, device="cuda:0", dtype=torch.uint8)
    flush = lambda: flush_buf.fill_(1)  # noqa: E731
    out = {}
    for name, with_bwd in (("small_model", False), ("train_4k", True)):
        w = inputs.WORKLOADS[name]
        st = Step(w, w.L, seed=0, pack=False, bwd=with_bwd)
        st.run()
        ms = events_ms(torch, st.run, 9, flush)
        nbytes = fwd_bytes(w) + (bwd_bytes(w) if with_bwd else 0)
        out[f"{name}_cold"] = {"what": "forward+backward" if with_bwd else "forward",
                               "ms": round(ms, 4), "bytes": nbytes,
                               "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                               "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        st.free()
    del flush_buf
    torch.cuda.empty_cache()
    return out


def fwd_pair(torch, w, reps=9, **kw):
    """Median forward milliseconds of w at its L and at L = 0, launched alternately."""
    a = Step(w, w.L, seed=0, pack=False, bwd=False, **kw)
    b = Step(w, 0, seed=0, pack=False, bwd=False)
    a.run()
    b.run()
    ta, tb = [], []
    for _ in range(reps):
        ta.append(events_ms(torch, a.run, 1))
        tb.append(events_ms(torch, b.run, 1))
    a.free()
    b.free()
    ta.sort()
    tb.sort()
    return ta[reps // 2], tb[reps // 2]


def aux_measurements(torch, inputs):
    w = inputs.WORKLOADS["layer_1p5b_8k"]
    fl, f0 = fwd_pair(torch, w)
    out = {"layer_1p5b_8k": {
        "fwd_ms": round(fl, 4), "fwd_ms_L0": round(f0, 4),
        "fwd_tflops": round(fwd_flops(w) / (fl * 1e-3) / 1e12, 1),
        "overhead_fwd": round((fl - f0) / f0, 4),
        "overhead_fwd_pages_convention": round((fl - f0) / fl, 4),
        "eta": round(depth_eta(w), 4)}}
    out.update(cold_rates(torch, inputs))
    return out


# The pages' own figures for the workloads of --suite pages (README "Kernel Efficiency"
# tables: A100, bf16, forward+backward, FlashAttention-2 vs MoDA Triton kernels, in ms, and
# the extra time they print).  Context only: other hardware and other kernels.
PAGES_A100 = {
    "table2_T4096": (7.970, 10.750, 0.2586), "table2_T8192": (28.700, 35.427, 0.1899),
    "table2_T16384": (116.700, 127.661, 0.0859), "table2_T32768": (459.854, 480.914, 0.0438),
    "table2_T65536": (1831.668, 1883.026, 0.0273), "table2_G2": (28.982, 39.741, 0.2707),
    "table2_G4": (58.071, 68.939, 0.1576), "table2_G16": (233.700, 244.900, 0.0457),
    "table2_G32": (467.107, 480.767, 0.0284), "table2_L128": (116.700, 138.224, 0.1557),
    "table2_L256": (116.700, 167.958, 0.3052),
}


def suite_pages(torch, inputs, steps, warmup):
    """One line per workload of the pages' efficiency tables: forward+backward at L and at
    L = 0 through the same entry points (depth rows already packed), and the depth-scan
    ablation at the Table 7 shape.  "ms" is the median of separately timed steps, so that
    one host stall between two launches does not move it; "ms_mean" is the average of
    back-to-back steps, and the kernel times are averages over those."""
    for name, w in inputs.PAGE_WORKLOADS.items():
        st = Step(w, w.L, seed=0, pack=False)
        ms_mean, k, _ = st.timed(steps, warmup)
        ms = events_ms(torch, st.run, max(steps, 5))
        st.free()
        s0 = Step(w, 0, seed=0, pack=False)
        ms0_mean, k0, _ = s0.timed(steps, warmup)
        ms0 = events_ms(torch, s0.run, max(steps, 5))
        s0.free()
        fl = 3.5 * fwd_flops(w)
        fwd, fwd0 = k["fwd"]["avg_ms"], k0["fwd"]["avg_ms"]
        line = {
            "metric": "MoDA fwd+bwd TFLOP/s bf16 (pages' kernel workload)",
            "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "T": w.T, "d": w.d,
                       "L": w.L, "G": w.G},
            "ms": round(ms, 4), "ms_L0": round(ms0, 4), "ms_mean": round(ms_mean, 4),
            "ms_L0_mean": round(ms0_mean, 4), "fwd_ms": round(fwd, 4),
            "fwd_ms_L0": round(fwd0, 4),
            "fwd_tflops": round(fwd_flops(w) / (fwd * 1e-3) / 1e12, 2),
            "frac_mfma_fwd_bwd": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "overhead_fwd_bwd": round((ms - ms0) / ms0, 4),
            "overhead_fwd_bwd_pages_convention": round((ms - ms0) / ms, 4),
            "overhead_fwd": round((fwd - fwd0) / fwd0, 4),
            "eta": round(depth_eta(w), 4),
            "kernels_ms": {n: round(v["avg_ms"], 4) for n, v in k.items()},
        }
        if name in PAGES_A100:
            fa2, moda, extra = PAGES_A100[name]
            line["pages_a100_context"] = {"fa2_ms": fa2, "moda_ms": moda, "extra_time": extra}
        print(json.dumps(line), flush=True)
    suite_ablation(torch, inputs)


def suite_ablation(torch, inputs):
    """The kernel ablation of depth-KV layouts at the Table 7 shape (T=1024, G=8, L=64):
    the forward with each choice of the depth rows a query block scores, one line each,
    10 launches of each scan in order (scan 0, then 1, then 2; the last 9 timed)."""
    w = inputs.PAGE_WORKLOADS["table7"]
    st = Step(w, w.L, seed=0, pack=False, bwd=False)
    mb, x = st.mb, st.x
    labels = {0: "own tokens per query block (library)", 1: "whole query chunk (chunk-aware)",
              2: "all T*L rows (flat layout, no chunking)"}
    for scan in (0, 1, 2):
        run = lambda: mb.moda_fwd_depth_scan(st.p, scan, x["Q"], x["K"], x["V"], st.Kd,  # noqa: E731
                                             st.Vd, st.O, st.lse)
        run()
        ms = events_ms(torch, run, 9)
        eta = depth_eta(w, scan)
        print(json.dumps({
            "metric": "MoDA forward ms, depth-scan ablation (Table 7 shape)", "value": round(ms, 4),
            "unit": "ms", "config": {"workload": "table7", "scan": scan, "layout": labels[scan]},
            "eta": round(eta, 6),
            # K and V rows of d bf16 scored once per 32x32 block of (rows, queries)
            "depth_bytes_read_GB": round(4 * w.d * w.B * w.Hq * w.T * w.L / (32 * eta) / 1e9, 3),
            "pages_table7_context_ms": {0: 1.460, 1: 6.286, 2: 13.102}[scan]}), flush=True)
    st.free()


# Decode and append are timed as a decoding loop issues them: LOOP_CALLS calls back to back
# between two events, per call (the host's launch latency then overlaps the GPU work); the
# single-call time, which includes that latency, is reported beside it.
LOOP_CALLS = 20


def suite_ceiling(torch, launch_ms=20.0, timed=10):
    """The chip's sustained bf16 matrix-core rate: the probe kernel of libmoda_probe.so (four
    independent 32x32x16 MFMA chains per wave, no memory traffic in its loop) on every CU, at
    one and two waves per SIMD, with fixed B operands (a loop of MFMAs and loop control only)
    and with one operand register changed after each MFMA (one vector instruction each).  Each setting runs
    3 untimed launches, then `timed` launches of about launch_ms each back to back; the line
    gives their median rate and the mean shader clock (s_memtime ticks over 100 MHz
    s_memrealtime ticks of each workgroup)."""
    import ctypes
    import statistics
    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_moda_amd", "libmoda_probe.so"))
    lib.moda_probe_mfma.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.moda_probe_mfma.restype = ctypes.c_int
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream
    flop_per_iter_wave = 4 * 32768                       # four MFMAs of 32x32x16
    for wps in (1, 2):
        wg = ncu * wps
        # Iterations for about launch_ms at the nominal peak.
        iters = int(launch_ms * 1e-3 * MFMA_BF16_PEAK_TFLOPS * 1e12
                    / (wg * 4 * flop_per_iter_wave)) // 4 * 4   # the probe unrolls by 4
        sink = torch.empty(wg * 256, device="cuda:0", dtype=torch.float32)
        clocks = torch.zeros(2 * wg, device="cuda:0", dtype=torch.int64)
        for vary in (0, 1):
            def launch():
                rc = lib.moda_probe_mfma(wg, iters, wps, vary, sink.data_ptr(), clocks.data_ptr(),
                                         stream)
                if rc != 0:
                    raise RuntimeError(f"moda_probe_mfma failed ({rc})")
            for _ in range(3):
                launch()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(timed + 1)]
            ev[0].record()
            for i in range(timed):
                launch()
                ev[i + 1].record()
            torch.cuda.synchronize()
            c = clocks.view(wg, 2).double()
            ghz = float((c[:, 0] / c[:, 1]).mean()) * 0.1   # the last launch's clock
            ms = statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(timed))
            tf = wg * 4 * iters * flop_per_iter_wave / (ms * 1e-3) / 1e12
            print(json.dumps({
                "metric": "sustained bf16 MFMA rate (probe, no memory traffic)",
                "value": round(tf, 1), "unit": "TFLOP/s",
                "frac_nominal": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "clock_GHz": round(ghz, 3), "waves_per_simd": wps,
                "operands": "changing" if vary else "fixed", "ms_per_launch": round(ms, 3),
                "launches": timed, "cus": ncu}), flush=True)
        del sink, clocks


def suite_decode(torch, inputs, steps, same_cache=True):
    """Decode, depth append and the variants at the 64K shape (B=1, Hq=16, Hk=8, d=128,
    L=24), each against its roofline."""
    from transformer_attention_moda_amd import binding as mb
    w = inputs.WORKLOADS["long_64k"]
    # A decoding loop calls the operator once per layer, each call on that layer's own cache.
    # The timed calls therefore cycle through several K/V caches, at least 1 GiB in all, so
    # that none is still in the 256 MB last-level cache when its turn comes round again. The
    # time of back-to-back calls on one cache, which that cache partly serves, is reported
    # beside it.
    for B, window in ((1, 0), (16, 0), (1, 4)):
        wb = w.with_(B=B)
        x = inputs.make(wb, seed=0, device="cuda:0", names=("Q", "K", "V", "Kd", "Vd"))
        kv_bytes = 2 * 2 * B * w.Hk * w.T * w.d
        ncache = max(2, -(-(1 << 30) // kv_bytes))
        caches = [(x["K"], x["V"])] + [
            tuple(inputs.make(wb, seed=i, device="cuda:0", names=("K", "V")).values())
            for i in range(1, ncache)]
        q = x["Q"][:, :, -1].contiguous()
        p = mb.problem(B, w.Hq, w.Hk, w.T, w.d, w.L, w.scale, window=window)
        O = torch.empty_like(q)
        lse = torch.empty((B, w.Hq), device="cuda:0")
        ws = torch.empty(mb.moda_decode_workspace_bytes(p), device="cuda:0", dtype=torch.uint8)
        calls = [lambda K=K, V=V: mb.moda_decode(p, w.T - 1, q, K, V, x["Kd"], x["Vd"], O, lse, ws)
                 for K, V in caches]
        turn = [0]

        def next_call():
            calls[turn[0] % ncache]()
            turn[0] += 1
        for c in calls:
            c()
        ms_one = events_ms(torch, next_call, max(steps, 9))
        ms = events_ms(torch, lambda: [next_call() for _ in range(LOOP_CALLS)], 9) / LOOP_CALLS
        ms_same = (events_ms(torch, lambda: [calls[0]() for _ in range(LOOP_CALLS)], 9) / LOOP_CALLS
                   if same_cache else None)
        # One call per cache captured in a HIP graph and replayed in turn: no host-side work.
        graphs = []
        for c in calls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                c()
            graphs.append(g)
        gturn = [0]

        def next_replay():
            graphs[gturn[0] % ncache].replay()
            gturn[0] += 1
        ms_graph = events_ms(torch, next_replay, max(steps, 9))
        del graphs
        W = window or w.L
        nbytes = 2 * (2 * B * w.Hk * w.T * w.d + 2 * B * w.Hk * W * w.d + 2 * B * w.Hq * w.d)
        print(json.dumps({
            "metric": "MoDA decode step GB/s (one new token, 64K cache)",
            "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "config": {"workload": "decode_64k", "B": B, "Hq": w.Hq, "Hk": w.Hk, "T": w.T,
                       "d": w.d, "L": w.L, "window": window, "caches_in_turn": ncache},
            "us": round(ms * 1e3, 2), "us_single_call": round(ms_one * 1e3, 2),
            "us_graph_replay": round(ms_graph * 1e3, 2),
            "us_same_cache": round(ms_same * 1e3, 2) if ms_same else None, "bytes": nbytes,
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
        del x, caches, calls, q, O, lse, ws
        torch.cuda.empty_cache()
    # The append, likewise, takes its layers in turn, each into its own slot.
    nlay = 4
    layers = [inputs.normal((w.B, w.Hk, w.T, w.d), seed=i, tensor="layers_K", device="cuda:0")
              for i in range(nlay)]
    packed = torch.empty((w.B, w.Hk, w.T * w.L, w.d), device="cuda:0", dtype=torch.bfloat16)
    p = mb.problem(w.B, w.Hk, w.Hk, w.T, w.d, w.L, 1.0)
    aturn = [0]

    def next_append():
        i = aturn[0] % nlay
        mb.moda_depth_append(p, layers[i], i, 0, packed)
        aturn[0] += 1
    for _ in range(nlay):
        next_append()
    ms_one = events_ms(torch, next_append, 9)
    ms = events_ms(torch, lambda: [next_append() for _ in range(LOOP_CALLS)], 9) / LOOP_CALLS
    nbytes = 2 * layers[0].numel() * 2
    print(json.dumps({"metric": "MoDA depth-cache append GB/s (one layer, 64K tokens)",
                      "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                      "config": {"workload": "append_64k", "B": w.B, "Hk": w.Hk, "T": w.T,
                                 "d": w.d, "L": w.L, "layers_in_turn": nlay},
                      "us": round(ms * 1e3, 2), "us_single_call": round(ms_one * 1e3, 2),
                      "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
    del layers, packed
    torch.cuda.empty_cache()
    st = Step(w, w.L, seed=0, pack=False, causal=False)
    ms, k, _ = st.timed(max(3, steps // 3), 1)
    st.free()
    pairs = w.T * w.T + w.T * w.L
    fl = 3.5 * 4.0 * w.d * w.B * w.Hq * pairs
    print(json.dumps({"metric": "MoDA non-causal fwd+bwd TFLOP/s bf16 (64K shape)",
                      "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                      "config": {"workload": "long_64k_noncausal"}, "ms": round(ms, 3),
                      "fwd_ms": round(k["fwd"]["avg_ms"], 3),
                      "frac_mfma": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}),
          flush=True)
    fw4, f0 = fwd_pair(torch, w, reps=5, window=4)
    print(json.dumps({"metric": "MoDA windowed forward ms (last 4 of 24 depth slots, 64K shape)",
                      "value": round(fw4, 4), "unit": "ms",
                      "config": {"workload": "long_64k_window4"}, "fwd_ms_L0": round(f0, 4),
                      "overhead_fwd": round((fw4 - f0) / f0, 4),
                      "eta": round(depth_eta(w, window=4), 4)}), flush=True)



def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from transformer_attention_moda_amd import binding, inputs
    binding.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe_mib > 0:
        # A kernel of known traffic for scaling hardware byte counters: the packer with
        # L = 1 is a plain copy (reads and writes copy_probe_mib MiB once).
        n = (args.copy_probe_mib << 20) // 256
        src = torch.ones((1, 1, 1, n, 128), device="cuda:0", dtype=torch.bfloat16)
        dst = torch.empty((1, 1, n, 128), device="cuda:0", dtype=torch.bfloat16)
        torch.cuda.synchronize()
        binding.moda_pack_depth(binding.problem(1, 1, 1, n, 128, 1, 1.0), src, dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if args.suite == "pages":
        suite_pages(torch, inputs, args.steps, args.warmup)
        return
    if args.suite == "decode":
        suite_decode(torch, inputs, args.steps, same_cache=not args.no_same_cache)
        return
    if args.suite == "ablation":
        suite_ablation(torch, inputs)
        return
    if args.suite == "ceiling":
        suite_ceiling(torch)
        return
    w = inputs.WORKLOADS.get(args.workload) or inputs.PAGE_WORKLOADS[args.workload]

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
        if bound is None:   # a kernel without a roofline of its own (the split pass's reduce)
            return {"bound": None}
        if bound == "mfma":
            ach, peak, unit = amount / (k["avg_ms"] * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = amount / (k["avg_ms"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4)}

    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["per_step"])
    roofline = dict(roof(dom, kernels[dom], w), traffic=traffic_for(dom, w.name), kernel=dom,
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
    step.free()
    aux = None if args.no_aux else aux_measurements(torch, inputs)

    out = {
        "metric": ("MoDA fwd+bwd TFLOP/s bf16 at T=64K (% MFMA peak); overhead vs own L=0 path"
                   if args.workload == "long_64k" else
                   f"MoDA fwd+bwd TFLOP/s bf16, {args.workload} (% MFMA peak); overhead vs own L=0 path"),
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
        "eta": round(depth_eta(w), 4),
        "cpu_baseline": cpu,
        "aux": aux,
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
