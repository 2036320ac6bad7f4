// Depth-KV layout packer: layer-major [L, B, Hk, T, d] -> token-major
// [B, Hk, T*L, d], packed row t*L + l = layers[l, b, kv, t].
//
// In the natural per-layer layout the L entries of one token lie T*d elements
// apart, which defeats coalesced reads in the attention kernel; the flattened
// token-major layout puts a token's L depth rows in one contiguous block
// ("Mixture-of-Depths Attention", arXiv 2603.15619, paper summary,
// "Hardware-Efficient Implementation", natural-layout paragraph and
// "Flash-compatible depth-KV layout").  The kernel is a bitwise copy bound by
// HBM bandwidth.  Lane i owns 16-byte chunk i of the [B*Hk*T, row] source rows and
// walks the L layers: for each layer a workgroup reads 256 consecutive chunks (one
// contiguous span) and writes them as depth row l of their tokens.  Its index
// division happens once, not per layer; loads and stores are non-temporal (every
// byte is touched once).
#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int PACK_THREADS = 256;
constexpr int PACK_UNROLL = 8;   // layers in flight per lane

__global__ __launch_bounds__(PACK_THREADS) void pack_kernel(const u32x4* __restrict__ in,
                                                            u32x4* __restrict__ out, int L,
                                                            int64_t chunks, int64_t cpr)
{
    // chunks = B*Hk*T*cpr source chunks per layer; chunk i is chunk i % cpr of row i / cpr.
    for (int64_t i = (int64_t)blockIdx.x * PACK_THREADS + threadIdx.x; i < chunks;
         i += (int64_t)gridDim.x * PACK_THREADS) {
        const int64_t row = i / cpr, ch = i - row * cpr;
        const u32x4* src = in + i;
        u32x4* dst = out + row * L * cpr + ch;
        int l = 0;
        for (; l + PACK_UNROLL <= L; l += PACK_UNROLL) {
            u32x4 v[PACK_UNROLL];
#pragma unroll
            for (int u = 0; u < PACK_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + (l + u) * chunks);
#pragma unroll
            for (int u = 0; u < PACK_UNROLL; ++u) __builtin_nontemporal_store(v[u], dst + (l + u) * cpr);
        }
        for (; l < L; ++l) __builtin_nontemporal_store(__builtin_nontemporal_load(src + l * chunks), dst + l * cpr);
    }
}

}  // namespace

hipError_t launch_pack_depth(int64_t L, int64_t B, int64_t Hk, int64_t T, int64_t row_bytes,
                             const void* layers, void* packed, hipStream_t st)
{
    const int64_t cpr = row_bytes / 16;
    const int64_t chunks = B * Hk * T * cpr;
    int64_t blocks = (chunks + PACK_THREADS - 1) / PACK_THREADS;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    timing_begin("pack", st);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, st,
                       (const u32x4*)layers, (u32x4*)packed, (int)L, chunks, cpr);
    timing_end(st);
    return hipGetLastError();
}

}  // namespace moda
