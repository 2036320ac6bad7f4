"""Static checks of the kernels' gfx950 assembly (built here with hipcc; no GPU).

Cross-lane instructions -- the matrix-core products (v_mfma_*), the transposed LDS reads
(ds_read_b64_tr_b16) and the half-wave swaps (v_permlane32_swap) -- combine values of
every lane of a wave, so they are only meaningful with all 64 lanes active.  A loop whose
trip count the compiler cannot prove wave-uniform is built as a divergent loop: lanes
that leave are removed from EXEC (s_andn2_b64 exec, exec, ...) while the others go on.
Such a loop must hold none of those instructions.  Every loop of every kernel that
carries them has wave-uniform bounds by construction (wave index through readfirstlane,
bounds from kernel arguments and that index); this test keeps it so in the compiled
code.  A control kernel with a lane-dependent trip count around an MFMA shows that the
check finds such a loop.

The kernels also keep (almost) nothing in scratch memory: a spilled register is a memory
round trip, and in a tile loop it stalls every wave that reloads it.  Each kernel's
private segment size is compared with a table: zero, except for two instances whose
few spilled values live outside their loops."""
import os
import re
import shutil
import subprocess
from collections import defaultdict
from concurrent.futures import ThreadPoolExecutor

import pytest

from transformer_attention_moda_amd import build

CROSS_LANE = ("v_mfma", "ds_read_b64_tr_b16", "v_permlane32_swap")
KERNEL_SOURCES = ("fwd_bf16.hip", "bwd_bf16.hip", "decode.hip")
ALL_SOURCES = KERNEL_SOURCES + ("pack.hip", "rowwise.hip")
# Scratch bytes per lane allowed, by mangled-name fragment (every other kernel: none).
#   the windowed d = 128, 8-wave forward: a few prologue values, outside its loops;
#   the d = 64 bwd_dkdv at two waves per SIMD (256 registers): outside its tile loop.
SCRATCH_ALLOWED = {"fwd_bf16_kernelILi128ELi8ELb1E": 12, "bwd_dkdv_kernelILi64ELi8ELi2ELb0E": 32}

pytestmark = pytest.mark.skipif(shutil.which(build.HIPCC) is None and
                                not os.path.exists(build.HIPCC), reason="hipcc not found")


def device_asm(src_path, out_dir):
    out = os.path.join(out_dir, os.path.basename(src_path) + ".s")
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-Wall")]
    subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", src_path, "-o", out],
                   check=True, capture_output=True)
    return open(out).read()


def functions(asm):
    """(name, lines) of every kernel in a device assembly file."""
    cur, lines = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur, lines = m.group(1), []
        if cur:
            lines.append(line)
        if cur and line.startswith(".Lfunc_end"):
            yield cur, lines
            cur = None


def divergent_loops_with_cross_lane_ops(asm):
    """[(kernel, loop header, count)] for loops (as the compiler annotates them) that
    remove lanes from EXEC to leave and hold cross-lane instructions."""
    found = []
    for name, lines in functions(asm):
        loops, cur = defaultdict(list), None
        for line in lines:
            m = re.match(r"^(\.LBB\w+):\s*(;.*)?$", line)
            if m:
                note = m.group(2) or ""
                inner = re.search(r"Header=(BB\w+)", note)
                cur = m.group(1)[2:] if "Loop Header" in note else (inner.group(1) if inner else None)
            elif cur:
                loops[cur].append(line.strip())
        for header, body in loops.items():
            if any(re.match(r"s_andn2_b64\s+exec, exec", s) for s in body):
                n = sum(any(op in s for op in CROSS_LANE) for s in body)
                if n:
                    found.append((name, header, n))
    return found


CONTROL = r"""
#include <hip/hip_runtime.h>
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ void lane_dependent_trip_count(float* out, int n)
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < (int)(threadIdx.x % 7) + n; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(1.0f, (float)i, acc, 0, 0, 0);
    out[threadIdx.x] = acc[0];
}
"""


def test_detector_finds_a_divergent_loop_around_an_mfma(tmp_path):
    src = tmp_path / "control.hip"
    src.write_text(CONTROL)
    found = divergent_loops_with_cross_lane_ops(device_asm(str(src), str(tmp_path)))
    assert found and "lane_dependent_trip_count" in found[0][0], found


@pytest.fixture(scope="module")
def library_asm(tmp_path_factory):
    """Device assembly of every kernel source of the library, by file name."""
    out = str(tmp_path_factory.mktemp("asm"))
    paths = [os.path.join(build.CSRC, s) for s in ALL_SOURCES]
    with ThreadPoolExecutor(len(paths)) as ex:
        return dict(zip(ALL_SOURCES, ex.map(lambda p: device_asm(p, out), paths)))


def test_no_kernel_runs_cross_lane_instructions_in_a_divergent_loop(library_asm):
    kernels = 0
    for src in KERNEL_SOURCES:
        asm = library_asm[src]
        kernels += sum(1 for _ in functions(asm))
        found = divergent_loops_with_cross_lane_ops(asm)
        assert not found, (src, found)
    assert kernels >= 16, kernels   # every template instance was seen


def scratch_bytes(asm):
    """{kernel: private segment bytes per lane} from the kernel descriptors."""
    sizes, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^\s*\.amdhsa_kernel\s+(\S+)", line)
        if m:
            cur = m.group(1)
        m = re.match(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", line)
        if m and cur:
            sizes[cur] = int(m.group(1))
    return sizes


def test_kernels_keep_no_scratch_beyond_the_listed_instances(library_asm):
    sizes = {}
    for src in ALL_SOURCES:
        sizes.update(scratch_bytes(library_asm[src]))
    assert len(sizes) >= 30, sorted(sizes)   # every kernel descriptor was read
    for frag in SCRATCH_ALLOWED:
        assert any(frag in k for k in sizes), frag   # the exceptions still name real kernels
    over = {}
    for name, n in sizes.items():
        allowed = max([v for f, v in SCRATCH_ALLOWED.items() if f in name], default=0)
        if n > allowed:
            over[name] = (n, allowed)
    assert not over, over
