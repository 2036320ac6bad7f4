// Depth-KV layout packer: layer-major [L, B, Hk, T, d] -> token-major
// [B, Hk, T*L, d], packed row t*L + l = layers[l, b, kv, t]; and its
// append form, one layer's entries for a token range written into one slot of
// an existing packed cache (the DepthKVCache role of the "moda-attention 0.1.0"
// PyPI page's architecture list: contiguous depth KV storage across layers).
//
// In the natural per-layer layout the L entries of one token lie T*d elements
// apart, which defeats coalesced reads in the attention kernel; the flattened
// token-major layout puts a token's L depth rows in one contiguous block
// ("Mixture-of-Depths Attention", arXiv 2603.15619, paper summary,
// "Hardware-Efficient Implementation", natural-layout paragraph and
// "Flash-compatible depth-KV layout").  The kernel is a bitwise copy bound by
// HBM bandwidth.  It walks the packed rows in output order, so that a workgroup's
// stores are one contiguous span (writes are the slower side of a copy on this chip),
// and reads each 16-byte chunk from its layer: a token's row of one layer is 256
// contiguous bytes.  Four chunks are in flight per lane, and the grid covers the whole
// tensor in one pass; loads and stores are non-temporal (every byte is touched once).
#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int PACK_THREADS = 256;
constexpr int PACK_UNROLL = 4;   // chunks in flight per lane

__global__ __launch_bounds__(PACK_THREADS) void pack_kernel(const u32x4* __restrict__ in,
                                                            u32x4* __restrict__ out, int L,
                                                            int64_t chunks, int64_t cpr)
{
    // chunks = B*Hk*T*cpr source chunks per layer.  Packed chunk j, of packed row
    // pr = ((b*Hk + kv)*T + t)*L + l, is chunk (pr / L)*cpr + j % cpr of layer pr % L.
    const int64_t total = (int64_t)L * chunks;
    const int64_t stride = (int64_t)gridDim.x * PACK_THREADS * PACK_UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * PACK_THREADS * PACK_UNROLL + threadIdx.x;
         base < total; base += stride) {
        u32x4 v[PACK_UNROLL];
#pragma unroll
        for (int u = 0; u < PACK_UNROLL; ++u) {
            const int64_t j = base + u * PACK_THREADS;
            if (j < total) {
                const int64_t pr = j / cpr, ch = j - pr * cpr;
                const int64_t bt = pr / L;
                const int l = (int)(pr - bt * L);
                v[u] = __builtin_nontemporal_load(in + l * chunks + bt * cpr + ch);
            }
        }
#pragma unroll
        for (int u = 0; u < PACK_UNROLL; ++u) {
            const int64_t j = base + u * PACK_THREADS;
            if (j < total) __builtin_nontemporal_store(v[u], out + j);
        }
    }
}

// Append: chunk i of the [B*Hk*n, cpr] source rows goes to chunk i % cpr of depth row
// (t0 + r % n)*L + slot of block r / n, r = i / cpr.
__global__ __launch_bounds__(PACK_THREADS) void append_kernel(const u32x4* __restrict__ in,
                                                              u32x4* __restrict__ out,
                                                              int64_t chunks, int64_t cpr,
                                                              int64_t n, int64_t T, int64_t L,
                                                              int64_t t0, int64_t slot)
{
    for (int64_t i = (int64_t)blockIdx.x * PACK_THREADS + threadIdx.x; i < chunks;
         i += (int64_t)gridDim.x * PACK_THREADS) {
        const int64_t r = i / cpr, ch = i - r * cpr;
        const int64_t bkv = r / n, t = t0 + (r - bkv * n);
        __builtin_nontemporal_store(__builtin_nontemporal_load(in + i),
                                    out + ((bkv * T + t) * L + slot) * cpr + ch);
    }
}

}  // namespace

hipError_t launch_depth_append(int64_t B, int64_t Hk, int64_t T, int64_t L, int64_t row_bytes,
                               int64_t slot, int64_t t0, int64_t n, const void* layer,
                               void* packed, hipStream_t st)
{
    const int64_t cpr = row_bytes / 16;
    const int64_t chunks = B * Hk * n * cpr;
    int64_t blocks = (chunks + PACK_THREADS - 1) / PACK_THREADS;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    timing_begin("depth_append", st);
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, st,
                       (const u32x4*)layer, (u32x4*)packed, chunks, cpr, n, T, L, t0, slot);
    timing_end(st);
    return hipGetLastError();
}

hipError_t launch_pack_depth(int64_t L, int64_t B, int64_t Hk, int64_t T, int64_t row_bytes,
                             const void* layers, void* packed, hipStream_t st)
{
    const int64_t cpr = row_bytes / 16;
    const int64_t chunks = B * Hk * T * cpr;
    int64_t blocks = (L * chunks + PACK_THREADS * PACK_UNROLL - 1) / (PACK_THREADS * PACK_UNROLL);
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    timing_begin("pack", st);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, st,
                       (const u32x4*)layers, (u32x4*)packed, (int)L, chunks, cpr);
    timing_end(st);
    return hipGetLastError();
}

}  // namespace moda
