// Depth-KV layout packer: layer-major [L, B, Hk, T, d] -> token-major
// [B, Hk, T*L, d], packed row t*L + l = layers[l, b, kv, t].
//
// In the natural per-layer layout the L entries of one token lie T*d elements
// apart, which defeats coalesced reads in the attention kernel; the flattened
// token-major layout puts a token's L depth rows in one contiguous block
// ("Mixture-of-Depths Attention", arXiv 2603.15619, paper summary,
// "Hardware-Efficient Implementation", natural-layout paragraph and
// "Flash-compatible depth-KV layout").  The kernel is a bitwise copy bound by
// HBM bandwidth: every output 16-byte chunk is written once, in order, and
// every input row is read as whole 16-byte chunks.
#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

constexpr int PACK_THREADS = 256;
constexpr int PACK_UNROLL = 4;

__global__ __launch_bounds__(PACK_THREADS) void pack_kernel(const uint4* __restrict__ in,
                                                            uint4* __restrict__ out, int64_t L,
                                                            int64_t BHk, int64_t T, int64_t cpr,
                                                            int64_t total)
{
    // Output chunk o = ((bkv * T + t) * L + l) * cpr + ch.
    const int64_t stride = (int64_t)gridDim.x * PACK_THREADS * PACK_UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * PACK_THREADS * PACK_UNROLL + threadIdx.x;
         base < total; base += stride) {
        uint4 v[PACK_UNROLL];
        int64_t oi[PACK_UNROLL];
#pragma unroll
        for (int u = 0; u < PACK_UNROLL; ++u) {
            const int64_t o = base + (int64_t)u * PACK_THREADS;
            oi[u] = o;
            if (o < total) {
                const int64_t ch = o % cpr, r = o / cpr;
                const int64_t l = r % L, tt = r / L;         // tt = bkv * T + t
                v[u] = in[((l * BHk) * T + tt) * cpr + ch];
            }
        }
#pragma unroll
        for (int u = 0; u < PACK_UNROLL; ++u)
            if (oi[u] < total) out[oi[u]] = v[u];
    }
}

}  // namespace

hipError_t launch_pack_depth(int64_t L, int64_t B, int64_t Hk, int64_t T, int64_t row_bytes,
                             const void* layers, void* packed, hipStream_t st)
{
    const int64_t cpr = row_bytes / 16;
    const int64_t total = B * Hk * T * L * cpr;
    const int64_t per_block = (int64_t)PACK_THREADS * PACK_UNROLL;
    int64_t blocks = (total + per_block - 1) / per_block;
    if (blocks > 256 * 64) blocks = 256 * 64;
    timing_begin("pack", st);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, st,
                       (const uint4*)layers, (uint4*)packed, L, B * Hk, T, cpr, total);
    timing_end(st);
    return hipGetLastError();
}

}  // namespace moda
