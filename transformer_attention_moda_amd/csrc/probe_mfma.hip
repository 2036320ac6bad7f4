// Sustained bf16 matrix-core rate of the chip, for context beside the attention kernels'
// roofline figures (which are quoted against the nominal 2.4 GHz peak).  Not part of the
// operator: it is built into its own library, libmoda_probe.so.
//
// Every wave issues NCH independent chains of 32x32x16 bf16 MFMAs (fp32 accumulate) on
// register operands, UNROLL rounds per loop iteration, with no memory traffic in the loop.
// With `vary` one B-operand register of each MFMA has its mantissa bits flipped after use
// (one vector instruction per MFMA), so that the matrix cores see changing data as in real
// kernels; without it the loop holds MFMAs and loop control only.  Wave 0 of each
// workgroup records the shader-clock counter (s_memtime) and the fixed 100 MHz counter
// (s_memrealtime) before and after its loop, so the host can state the clock the chip ran at.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int NCH = 4;      // independent accumulator chains per wave
constexpr int UNROLL = 4;   // MFMA rounds per loop iteration

// LDS reserved per workgroup so that exactly WPS 4-wave workgroups fit on a CU (160 KiB):
// one per CU at 96 KiB, two at 72 KiB.  A grid of WPS workgroups per CU then puts WPS waves
// on every SIMD.
template <int WPS>
constexpr int kLdsWords = (WPS == 1 ? 96 : 72) * 1024 / 4;

template <int WPS, bool VARY>
__global__ __launch_bounds__(256, WPS) void mfma_probe_kernel(int64_t rounds, float* sink,
                                                              uint64_t* clocks)
{
    __shared__ float lds[kLdsWords<WPS>];
    const int lane = threadIdx.x & 63;
    lds[threadIdx.x * (kLdsWords<WPS> / 256)] = (float)lane;
    // Nonzero, lane-dependent operands (finite bf16 values of moderate size).
    i32x4 ai, bi[NCH];
#pragma unroll
    for (int k = 0; k < 4; ++k) ai[k] = 0x3f803f80 ^ ((lane * 0x00050003 + k * 0x00110007) & 0x007f007f);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            bi[c][k] = 0x3e803e80 ^ ((lane * 0x00030005 + (c * 4 + k) * 0x00070011) & 0x007f007f);
    f32x16 acc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
    const bool rec = (threadIdx.x >> 6) == 0;
    uint64_t t0 = 0, r0 = 0;
    if (rec) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int64_t it = 0; it < rounds; ++it) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ai),
                                                                __builtin_bit_cast(bf16x8, bi[c]),
                                                                acc[c], 0, 0, 0);
                // One vector instruction per MFMA: flips the mantissa bits of one operand
                // register (values stay finite and of the same size).
                if constexpr (VARY) bi[c][u & 3] ^= 0x007f007f;
            }
        }
    }
    if (rec) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            clocks[2 * blockIdx.x] = t1 - t0;
            clocks[2 * blockIdx.x + 1] = r1 - r0;
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[c][j];
    __syncthreads();
    s += lds[((threadIdx.x + 1) & 255) * (kLdsWords<WPS> / 256)];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the products live
}

}  // namespace

// Launches `workgroups` 4-wave workgroups of the probe, each wave doing iters MFMA rounds of
// NCH = 4 MFMAs of 32x32x16 (32768 FLOP each); iters is rounded down to a multiple of 4.  waves_per_simd (1 or 2) sets how many workgroups share a CU
// (through their LDS reservation); a grid of waves_per_simd workgroups per CU fills the chip.
// sink: float[workgroups * 256]; clocks: uint64[2 * workgroups] (shader-clock ticks and
// 100 MHz ticks of each workgroup's wave 0).  Returns a hipError_t.
extern "C" int moda_probe_mfma(int64_t workgroups, int64_t iters, int waves_per_simd, int vary,
                               float* sink, uint64_t* clocks, void* stream)
{
    if (workgroups < 1 || workgroups > (int64_t(1) << 24) || iters < UNROLL || !sink ||
        !clocks || (waves_per_simd != 1 && waves_per_simd != 2))
        return (int)hipErrorInvalidValue;
    hipStream_t st = (hipStream_t)stream;
    const int64_t rounds = iters / UNROLL;
    const dim3 grid((unsigned)workgroups), block(256);
    if (waves_per_simd == 1) {
        if (vary) hipLaunchKernelGGL((mfma_probe_kernel<1, true>), grid, block, 0, st, rounds, sink, clocks);
        else hipLaunchKernelGGL((mfma_probe_kernel<1, false>), grid, block, 0, st, rounds, sink, clocks);
    } else {
        if (vary) hipLaunchKernelGGL((mfma_probe_kernel<2, true>), grid, block, 0, st, rounds, sink, clocks);
        else hipLaunchKernelGGL((mfma_probe_kernel<2, false>), grid, block, 0, st, rounds, sink, clocks);
    }
    return (int)hipGetLastError();
}
