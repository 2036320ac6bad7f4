"""bench.py's command line on the host: more than one GPU is refused before any GPU work,
with one JSON line that says so and a non-zero exit status."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_is_reported_only_for_the_profiled_workload():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.traffic_for("bwd_dkdv", "table2_T4096") is None   # never profiled
    assert bench.traffic_for("no_such_kernel", "long_64k") is None
    t = bench.traffic_for("bwd_dkdv", "long_64k")   # None once the sources change
    assert t is None or (t["fetch_bytes"] > 0 and t["bytes"] == t["fetch_bytes"] + t["write_bytes"])


def test_copy_probe_grid_follows_the_packer_launch():
    """The traffic summary finds bench.py's copy probe by the packer's grid; the launch
    constants are read from the packer's source so that a change there fails here."""
    import re
    sys.path.insert(0, ROOT)
    from transformer_attention_moda_amd import profile_summary
    src = open(os.path.join(ROOT, "transformer_attention_moda_amd", "csrc", "pack.hip")).read()
    threads = int(re.search(r"PACK_THREADS\s*=\s*(\d+)", src).group(1))
    unroll = int(re.search(r"PACK_UNROLL\s*=\s*(\d+)", src).group(1))
    cap = 1 << int(re.search(r"blocks\s*>\s*\(int64_t\(1\)\s*<<\s*(\d+)\)", src).group(1))
    for mib in (1, 1024, 3072, 1 << 16):
        chunks = (mib << 20) // 16
        blocks = min(-(-chunks // (threads * unroll)), cap)
        assert profile_summary.packer_grid(mib << 20) == blocks * threads


def test_mfma_probe_library_refuses_bad_arguments_on_the_host():
    """The ceiling suite's probe library is built beside libmoda.so and checks its arguments
    before any launch (no GPU call is made for a refused one)."""
    import ctypes
    path = os.path.join(ROOT, "transformer_attention_moda_amd", "libmoda_probe.so")
    assert os.path.exists(path), "run __graft_entry__.build() first"
    lib = ctypes.CDLL(path)
    f = lib.moda_probe_mfma
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    buf = ctypes.c_void_p(256)   # never dereferenced: every call below is refused first
    assert f(0, 10, 1, 0, buf, buf, None) != 0        # no workgroups
    assert f(256, 3, 1, 0, buf, buf, None) != 0       # fewer iterations than one unrolled round
    assert f(256, 10, 3, 0, buf, buf, None) != 0      # waves per SIMD must be 1 or 2
    assert f(256, 10, 1, 0, None, buf, None) != 0     # null output
