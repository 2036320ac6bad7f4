"""Per-kernel summaries of rocprofv3 output for libmoda's kernels.

    python -m transformer_attention_moda_amd.profile_summary counters <dir> [<dir> ...]
    python -m transformer_attention_moda_amd.profile_summary trace <dir> [--by-grid]
    python -m transformer_attention_moda_amd.profile_summary dispatches <dir> <kernel>
    python -m transformer_attention_moda_amd.profile_summary traffic <fetch_dir> <write_dir> \
        <probe_mib> <workload>
    python -m transformer_attention_moda_amd.profile_summary ablation <fetch_dir> <sq_dir> \
        <probe_mib>

`counters`: every `*counter_collection.csv` under the given rocprofv3 output
directories (one per --pmc pass); prints, per libmoda kernel, the mean over its
dispatches of each counter, the dispatch count and the mean duration, then the
derived rates below.  `trace`: every `*kernel_stats.csv` (rocprofv3
--kernel-trace --stats), the per-kernel call count and mean duration; with --by-grid, from
`*kernel_trace.csv`, the count and median duration per kernel and launch grid (one line per
problem size when a run launches a kernel at several).  `dispatches`: from
`*kernel_trace.csv`, every dispatch of the kernels whose name contains <kernel>, in launch
order, with its grid and duration.

Derived (when the counters are present): GRBM_GUI_ACTIVE / duration = the
graphics clock the counter ran at (summed over the chip's XCDs, so divided by
their count); SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CU_CYCLES or, failing that,
GRBM_GUI_ACTIVE x CUs per XCD) = fraction of CU cycles the matrix cores were busy;
SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS = bank-conflict cycles per LDS instruction
cycle; SQ_INSTS_* per wave = instruction mix; 4 x SQ_WAVE_CYCLES / SQ_BUSY_CU_CYCLES = mean
resident waves per CU (SQ_WAVE_CYCLES counts in units of 4 cycles).  `traffic`: HBM bytes
per launch from a FETCH_SIZE pass and a WRITE_SIZE pass (KiB per dispatch) of
`bench.py --copy-probe-mib <probe_mib>`, each scaled by what the same counter reads for
the probe (the packer with L = 1 copying probe_mib MiB: that many bytes read and written),
in the line format bench.py reads from profiles/traffic.txt.  `ablation`: the forward
dispatches of `bench.py --suite ablation` (the same kernel launched 10 times per depth scan,
scan 0, 1, 2 in that order) split into their three groups, with per scan the mean duration,
the HBM bytes fetched (FETCH_SIZE scaled by the copy probe as for `traffic`), the MFMA
instructions and the fraction of SIMD cycles the matrix cores were busy.  Nothing here runs on a GPU.
"""
from __future__ import annotations

import csv
import glob
import os
import re
import sys
from collections import defaultdict

XCDS = 8            # MI355X: 8 accelerator complex dies ...
CUS_PER_XCD = 32    # ... of 32 compute units each


def ours(kernel: str) -> bool:
    """A kernel of libmoda (namespace moda) or of its matrix-core rate probe."""
    return "moda" in kernel or "mfma_probe_kernel" in kernel


def short_name(kernel: str) -> str:
    """`void moda::(anonymous namespace)::fwd_bf16_kernel<128, 8, false>(...)` ->
    `fwd_bf16_kernel<128, 8, false>`."""
    k = kernel.split("(")[0] if "(" in kernel.split("<")[0] else kernel
    m = re.search(r"([A-Za-z_0-9]+_kernel(<[^()]*>)?)", kernel)
    return m.group(1) if m else k.strip()[-60:]


def _rows(pattern_dirs, suffix):
    for d in pattern_dirs:
        for path in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
            with open(path, newline="") as f:
                yield from csv.DictReader(f)


def counters(dirs):
    vals = defaultdict(lambda: defaultdict(list))     # kernel -> counter -> per dispatch
    dur = defaultdict(dict)                           # kernel -> dispatch -> ns
    for r in _rows(dirs, "counter_collection.csv"):
        name = r.get("Kernel_Name", "")
        if not ours(name):
            continue
        k = short_name(name)
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r.get("Counter_Name"))
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        s, e = r.get("Start_Timestamp"), r.get("End_Timestamp")
        if s and e:
            dur[k][key[0]] = float(e) - float(s)
    out = []
    for k in sorted(vals):
        c = {n: sum(v) / len(v) for n, v in vals[k].items()}
        ns = sum(dur[k].values()) / max(1, len(dur[k])) if dur[k] else None
        out.append(f"kernel {k}  dispatches={max(len(v) for v in vals[k].values())}"
                   + (f"  mean_duration_us={ns / 1e3:.1f}" if ns else ""))
        for n in sorted(c):
            out.append(f"  {n:32s} {c[n]:.6g}")
        g = c.get("GRBM_GUI_ACTIVE")
        if g and ns:
            out.append(f"  -> clock (GRBM_GUI_ACTIVE / {XCDS} XCDs / duration): "
                       f"{g / XCDS / ns:.3f} GHz")
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        cu = c.get("SQ_BUSY_CU_CYCLES") or (g / XCDS * XCDS * CUS_PER_XCD if g else None)
        if busy and cu:
            out.append(f"  -> matrix cores busy: {busy / cu:.3f} of CU cycles "
                       f"(SQ_VALU_MFMA_BUSY_CYCLES / "
                       f"{'SQ_BUSY_CU_CYCLES' if c.get('SQ_BUSY_CU_CYCLES') else 'GRBM_GUI_ACTIVE x CUs'})")
        if c.get("SQ_LDS_BANK_CONFLICT") is not None and c.get("SQ_ACTIVE_INST_LDS"):
            out.append(f"  -> LDS bank-conflict cycles per LDS-active cycle: "
                       f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_ACTIVE_INST_LDS']:.4f}")
        waves = c.get("SQ_WAVES")
        if waves:
            for n in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                      "SQ_INSTS_VMEM"):
                if n in c:
                    out.append(f"  -> {n} per wave: {c[n] / waves:.1f}")
        for n in ("SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"):
            if n in c and c.get("SQ_WAVE_CYCLES"):
                out.append(f"  -> {n} / SQ_WAVE_CYCLES: {c[n] / c['SQ_WAVE_CYCLES']:.3f}")
        if c.get("SQ_WAVE_CYCLES") and c.get("SQ_BUSY_CU_CYCLES"):
            out.append(f"  -> resident waves per CU: "
                       f"{4 * c['SQ_WAVE_CYCLES'] / c['SQ_BUSY_CU_CYCLES']:.2f}")
    return "\n".join(out)


# Sources whose hash marks a traffic line stale once a kernel changes.
SOURCES = {
    "pack": ["csrc/pack.hip", "csrc/common.hpp"],
    "fwd": ["csrc/fwd_bf16.hip", "csrc/common.hpp"],
}
for _k in ("bwd_pre", "bwd_depth", "bwd_dq", "bwd_dkdv"):
    SOURCES[_k] = ["csrc/bwd_bf16.hip", "csrc/common.hpp"]
LABELS = {"pack_kernel": "pack", "fwd_bf16_kernel": "fwd", "bwd_pre_kernel": "bwd_pre",
          "bwd_depth_kernel": "bwd_depth", "bwd_dq_kernel": "bwd_dq", "bwd_dkdv_kernel": "bwd_dkdv"}


def sources_sha(label):
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for src in SOURCES[label]:
        h.update(open(os.path.join(here, src), "rb").read())
    return h.hexdigest()[:16]


def packer_grid(nbytes):
    """Work-items of the packer's launch for a copy of nbytes with L = 1: 256-lane
    workgroups of 4 16-byte chunks per lane, at most 2^20 workgroups."""
    chunks = nbytes // 16
    return min((chunks + 1023) // 1024, 1 << 20) * 256


def traffic(fetch_dir, write_dir, probe_mib, workload):
    probe_bytes = probe_mib << 20
    probe_grid = packer_grid(probe_bytes)
    per = {}
    factors = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = defaultdict(list)
        probe = None
        for r in _rows([d], "counter_collection.csv"):
            if r["Counter_Name"] != counter or not ours(r["Kernel_Name"]):
                continue
            k = LABELS.get(short_name(r["Kernel_Name"]).split("<")[0])
            if k == "pack" and int(r["Grid_Size"]) == probe_grid and probe is None:
                probe = float(r["Counter_Value"])
                continue
            if k:
                vals[k].append(float(r["Counter_Value"]))
        if probe is None:
            raise SystemExit(f"no copy-probe dispatch (grid {probe_grid}) in {d}")
        factors[counter] = probe_bytes / (probe * 1024)
        for k, v in vals.items():
            per.setdefault(k, {})[counter] = (sum(v) / len(v) * 1024 * factors[counter], len(v))
    out = [f"# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE "
           f"(KiB per dispatch), scaled by a {probe_mib} MiB copy through the packer with L=1 in "
           f"the same run: factor {factors['FETCH_SIZE']:.4f} (FETCH_SIZE), "
           f"{factors['WRITE_SIZE']:.4f} (WRITE_SIZE).",
           "# sha: first 16 hex digits of sha256 over the listed sources; bench.py reports "
           "traffic only while it matches."]
    for k in ("pack", "fwd", "bwd_pre", "bwd_depth", "bwd_dq", "bwd_dkdv"):
        if k not in per:
            continue
        f, nf = per[k].get("FETCH_SIZE", (0.0, 0))
        wr, _ = per[k].get("WRITE_SIZE", (0.0, 0))
        srcs = ",".join("transformer_attention_moda_amd/" + x for x in SOURCES[k])
        out.append(f"kernel={k} workload={workload} sha={sources_sha(k)} sources={srcs} "
                   f"fetch_bytes={f:.4e} write_bytes={wr:.4e} launches_sampled={nf}")
    return "\n".join(out)


def trace_by_grid(dirs):
    durs = defaultdict(list)
    for r in _rows(dirs, "kernel_trace.csv"):
        if not ours(r.get("Kernel_Name", "")):
            continue
        grid = "x".join(r[f"Grid_Size_{a}"] for a in "XYZ")
        durs[(short_name(r["Kernel_Name"]), grid)].append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = []
    for (k, grid), v in sorted(durs.items()):
        v.sort()
        out.append(f"{k:44s} grid={grid:18s} calls={len(v):5d} median_us={v[len(v) // 2] / 1e3:10.1f} "
                   f"min_us={v[0] / 1e3:10.1f} max_us={v[-1] / 1e3:10.1f}")
    return "\n".join(out)


def ablation(fetch_dir, sq_dir, probe_mib):
    probe_bytes = probe_mib << 20
    probe_grid = packer_grid(probe_bytes)
    out = ["scan  launches  mean_us  fetch_GB  mfma_instr  matrix_busy"]
    per = {}
    factor = None
    for d in (fetch_dir, sq_dir):
        disp = defaultdict(dict)   # dispatch -> counter -> value, plus the duration
        for r in _rows([d], "counter_collection.csv"):
            name = r["Kernel_Name"]
            if "pack_kernel" in name and int(r["Grid_Size"]) == probe_grid and \
                    r["Counter_Name"] == "FETCH_SIZE" and factor is None:
                factor = probe_bytes / (float(r["Counter_Value"]) * 1024)
            if "fwd_bf16_kernel" not in name:
                continue
            k = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
            disp[k][r["Counter_Name"]] = float(r["Counter_Value"])
            disp[k]["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        ids = sorted(disp)
        n = len(ids) // 3
        for scan in range(3):
            group = [disp[i] for i in ids[scan * n:(scan + 1) * n]]
            for c in group[0]:
                per.setdefault(scan, {})[c] = sum(g[c] for g in group) / len(group)
            per[scan]["_n"] = len(group)
    for scan in range(3):
        c = per[scan]
        fetch = c.get("FETCH_SIZE", 0.0) * 1024 * (factor or float("nan")) / 1e9
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * c["SQ_BUSY_CU_CYCLES"]) \
            if c.get("SQ_BUSY_CU_CYCLES") else float("nan")
        out.append(f"{scan:4d}  {c['_n']:8d}  {c['_ns'] / 1e3:7.1f}  {fetch:8.3f}  "
                   f"{c.get('SQ_INSTS_MFMA', float('nan')):10.4g}  {busy:11.3f}")
    out.append(f"# FETCH_SIZE scale from the copy probe: {factor:.4f}" if factor else
               "# no copy probe found: fetch_GB not scaled")
    return "\n".join(out)


def dispatches(dirs, kernel):
    rows = [r for r in _rows(dirs, "kernel_trace.csv") if kernel in r.get("Kernel_Name", "")]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = []
    for i, r in enumerate(rows):
        grid = "x".join(r[f"Grid_Size_{a}"] for a in "XYZ")
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        out.append(f"{i:3d} {short_name(r['Kernel_Name']):44s} grid={grid:18s} us={us:10.1f}")
    return "\n".join(out)


def trace(dirs):
    out = []
    for r in _rows(dirs, "kernel_stats.csv"):
        if not ours(r.get("Name", "")):
            continue
        out.append(f"{short_name(r['Name']):44s} calls={r['Calls']:>5s} "
                   f"mean_us={float(r['AverageNs']) / 1e3:10.1f} "
                   f"min_us={float(r['MinNs']) / 1e3:10.1f} max_us={float(r['MaxNs']) / 1e3:10.1f}")
    return "\n".join(out)


def main(argv):
    if len(argv) < 2 or argv[0] not in ("counters", "trace", "traffic", "ablation", "dispatches"):
        print(__doc__)
        return 2
    if argv[0] == "ablation":
        print(ablation(argv[1], argv[2], int(argv[3])))
        return 0
    if argv[0] == "traffic":
        print(traffic(argv[1], argv[2], int(argv[3]), argv[4]))
    elif argv[0] == "dispatches":
        print(dispatches([argv[1]], argv[2]))
    else:
        if argv[0] == "counters":
            print(counters(argv[1:]))
        elif "--by-grid" in argv:
            print(trace_by_grid([d for d in argv[1:] if d != "--by-grid"]))
        else:
            print(trace(argv[1:]))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
