// MoDA decoding step, bfloat16 storage, for gfx950.
//
// One new query token per (batch, query head) at cache position pos attends to
// the cached sequence keys 0..pos (every cached key with the non-causal flag)
// and to its own depth rows pos*L + L-W .. pos*L + L-1: the forward's row at
// that token, computed for one token (the decoding cost of the paper summary's
// "Complexity Analysis", sequence part O(T d) and depth part O(L d) per layer,
// with a depth KV cache as the PyPI page's DepthKVCache keeps it).
//
// The work is one long, thin reduction, bound by the bytes of K and V it
// streams (4 d bytes per key, each used by the G heads of its group), so it is
// split over the sequence: for each (b, kv) the visible keys, then the depth
// rows, form 32-row blocks; with P waves on the (b, kv), wave p takes blocks
// p, p + P, p + 2P, ... (so that the waves of a unit read neighbouring blocks
// at about the same time) and keeps an online-softmax partial (running max m, sum l,
// unnormalised output o) for the G query heads of the group, held in the 32
// MFMA columns (columns past G repeat heads; their results are not written).
// Per block: S^T = K q^T on 32x32x16 bf16 MFMA with K rows loaded straight
// into registers as the A operand, the row mask, the online update, then
// o^T += V^T P^T with V staged in the wave's LDS slice for the transposed
// read; the next block's loads are issued while the current one computes.
// A second kernel merges the partials of each query row by the log-sum-exp
// rule and writes O (bf16) and lse (fp32).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

struct DecArgs {
    const uint16_t* q;    // [B, Hq, D]
    const uint16_t* K;    // [B, Hk, T, D]
    const uint16_t* V;
    const uint16_t* Kd;   // [B, Hk, T*L, D]
    const uint16_t* Vd;
    uint16_t* O;          // [B, Hq, D]
    float* lse;           // [B, Hq]
    float* part_o;        // [B*Hk][P][G][D] unnormalised outputs of the partials
    float* part_ml;       // [B*Hk][P][G][2] running max (score units) and sum
    int B, Hq, Hk, T, L, G, W;
    int pos;              // the query's token position in the cache
    int nseq;             // visible sequence keys 0..nseq-1
    int nblk_seq, nblk;   // 32-row blocks: the sequence ones first, then the depth ones
    int nsplit;           // workgroups per (b, kv)
    float c;              // scale * log2(e)
    float scale;
};

constexpr int DEC_NW = 4;   // waves per workgroup, each with its own partial

template <int D>
__global__ __launch_bounds__(DEC_NW * 64) void decode_partial_kernel(DecArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t vslot[DEC_NW][32 * D];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int col = lane & 31, hf = lane >> 5;
    const int bkv = blockIdx.x, kv = bkv % a.Hk, b = bkv / a.Hk;
    const int G = a.G, P = a.nsplit * DEC_NW;
    const int part = blockIdx.y * DEC_NW + w;
    const int nblk = a.nblk;   // this wave's blocks: part, part + P, ... below nblk

    bf16x8 qreg[D / 16];   // q^T columns as MFMA B operands, k-step si: d = 16 si + 8 hf ..
    {
        const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + kv * G + col % G) * D + 8 * hf;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) qreg[si] = __builtin_bit_cast(bf16x8, ld16(qrow + 16 * si));
    }
    f32x16 o[D / 32];
    zero(o);
    float m = -1e30f, l = 0.f;   // finite sentinel: a block with no visible row gives weights 0

    const int64_t kvbase = (int64_t)bkv * a.T;
    // Block i: its first row and the count of visible rows in it (>= 1).
    auto block_src = [&](int i, const uint16_t*& kbase, const uint16_t*& vbase, int& count) {
        if (i < a.nblk_seq) {
            kbase = a.K + (kvbase + 32 * (int64_t)i) * D;
            vbase = a.V + (kvbase + 32 * (int64_t)i) * D;
            count = min(32, a.nseq - 32 * i);
        } else {
            const int j = 32 * (i - a.nblk_seq);
            const int64_t r = (kvbase + a.pos) * a.L + (a.L - a.W) + j;
            kbase = a.Kd + r * D;
            vbase = a.Vd + r * D;
            count = min(32, a.W - j);
        }
    };
    constexpr int NK = D / 16;   // K load instructions per block
    bf16x8 kr[D / 16];
    uint16_t* const slot = vslot[w];
    auto issue_k = [&](int i) {   // rows past the block's visible ones repeat its last row
        const uint16_t *kb, *vb;
        int count;
        block_src(i, kb, vb, count);
        const uint16_t* krow = kb + (int64_t)min(col, count - 1) * D + 8 * hf;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) kr[si] = __builtin_bit_cast(bf16x8, ld16(krow + 16 * si));
    };
    auto issue_v = [&](int i) {
        const uint16_t *kb, *vb;
        int count;
        block_src(i, kb, vb, count);
        stage_rows<D>(slot, 32, vb, [&](int r) { return min(r, count - 1) * D; }, lane, 0, 1);
    };
    if (part < nblk) {
        issue_v(part);
        issue_k(part);
    }
    for (int i = part; i < nblk; i += P) {
        const bool more = i + P < nblk;
        const uint16_t *kb, *vb;
        int count;
        block_src(i, kb, vb, count);
        f32x16 s[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) s[0][j] = 0.f;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) s[0] = mfma32(kr[si], qreg[si], s[0]);
        if (more) issue_k(i + P);
        // register j holds row (j/4)*8 + 4 hf + j%4 of the block
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if ((j >> 2) * 8 + 4 * hf + (j & 3) >= count) s[0][j] = -INFINITY;
        softmax_update<D, 1>(s, m, l, o, a.c);
        if (more) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NK) : "memory");   // V of block i landed
        else wait_vmem();
        wave_lds_sync();
        pv_block<D>(slot, 0, s[0], o, lane);
        wave_lds_sync();
        if (more) issue_v(i + P);
    }

    // The partial of query head kv*G + col (columns past G repeat heads: not written).
    if (col < G) {
        const int64_t pi = ((int64_t)bkv * P + part) * G + col;
        float* orow = a.part_o + pi * D + 4 * hf;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *(float4*)(orow + 32 * db + 8 * jj) =
                    make_float4(o[db][4 * jj + 0], o[db][4 * jj + 1], o[db][4 * jj + 2], o[db][4 * jj + 3]);
        if (hf == 0) *(float2*)(a.part_ml + 2 * pi) = make_float2(m, l);
    }
}

constexpr int COMB_WAVES = 8;
constexpr int COMB_UNROLL = 8;   // partials whose loads are in flight per half-wave

// One workgroup per (query row (b, h), 32-wide slice of d): merge the group's P partials
// by the log-sum-exp rule for those 32 output elements.  All threads find the largest
// running max; each half-wave then accumulates partials hw, hw + 2 COMB_WAVES, ... (lane
// = element of the slice; loads of COMB_UNROLL partials in flight), and the half-waves'
// sums meet in LDS.  Spreading a row over D/32 workgroups spreads the partials' bytes
// over that many CUs.
template <int D>
__global__ __launch_bounds__(COMB_WAVES * 64) void decode_combine_kernel(DecArgs a)
{
    constexpr int SL = D / 32;   // slices per row
    constexpr int NH = 2 * COMB_WAVES;   // half-waves
    __shared__ float red[NH][33];
    __shared__ float wmax[COMB_WAVES];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int dl = lane & 31, hw = 2 * w + (lane >> 5);
    const int64_t row = blockIdx.x / SL;   // b*Hq + h
    const int slice = (int)(blockIdx.x % SL);
    const int h = (int)(row % a.Hq), b = (int)(row / a.Hq);
    const int kv = h / a.G, g = h % a.G;
    const int P = a.nsplit * DEC_NW;
    const int64_t first = ((int64_t)b * a.Hk + kv) * P * a.G + g;   // partial p at first + p*G
    float M = -1e30f;
    for (int p = threadIdx.x; p < P; p += COMB_WAVES * 64)
        M = fmaxf(M, a.part_ml[2 * (first + (int64_t)p * a.G)]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    if (lane == 0) wmax[w] = M;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < COMB_WAVES; ++i) M = fmaxf(M, wmax[i]);
    float lsum = 0.f, acc = 0.f;
    const int e = 32 * slice + dl;   // output element of this lane
    for (int p0 = hw; p0 < P; p0 += NH * COMB_UNROLL) {
        float2 ml[COMB_UNROLL];
        float ov[COMB_UNROLL];
#pragma unroll
        for (int u = 0; u < COMB_UNROLL; ++u) {
            const int p = min(p0 + NH * u, P - 1);
            const int64_t pi = first + (int64_t)p * a.G;
            ml[u] = *(const float2*)(a.part_ml + 2 * pi);
            ov[u] = a.part_o[pi * D + e];
        }
#pragma unroll
        for (int u = 0; u < COMB_UNROLL; ++u) {
            if (p0 + NH * u >= P) continue;
            const float wgt = fast_exp2((ml[u].x - M) * a.c);   // 0 for an empty partial
            lsum += wgt * ml[u].y;
            acc += wgt * ov[u];
        }
    }
    red[hw][dl] = acc;
    if (dl == 0) red[hw][32] = lsum;
    __syncthreads();
    if (threadIdx.x < 32) {
        float lt = 0.f, v = 0.f;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
            lt += red[j][32];
            v += red[j][dl];
        }
        const __bf16 o = (__bf16)(v / lt);
        a.O[row * D + e] = __builtin_bit_cast(uint16_t, o);
        if (slice == 0 && dl == 0) a.lse[row] = a.scale * M + __logf(lt);
    }
}

}  // namespace

DecodePlan plan_decode(const Shape& s, int64_t nseq)
{
    DecodePlan pl;
    const int64_t units = s.B * s.Hk;
    pl.nblk_seq = (nseq + 31) / 32;
    pl.nblk = pl.nblk_seq + (s.L > 0 ? (s.W + 31) / 32 : 0);
    // At d = 128 one wave per SIMD holds the partial kernel's registers, so one 4-wave
    // workgroup per CU: about 1024 waves over the chip's 256 CUs, in a single round. At
    // d = 64 three waves fit per SIMD, and about 2048 waves are launched. At least 2 blocks
    // per wave. The split count never decreases as nseq grows, so the largest nseq bounds
    // the workspace.
    const int64_t cap = std::max<int64_t>(1, (s.d == 128 ? 1024 : 2048) / (DEC_NW * units));
    pl.nsplit = std::min<int64_t>(cap, (pl.nblk + 2 * DEC_NW - 1) / (2 * DEC_NW));
    const int64_t parts = units * pl.nsplit * DEC_NW * s.G;
    pl.o_floats = parts * s.d;
    pl.ml_floats = parts * 2;
    return pl;
}

size_t decode_ws_bytes(const DecodePlan& pl)
{
    const size_t o = ((size_t)pl.o_floats * sizeof(float) + 255) & ~size_t(255);
    return o + (((size_t)pl.ml_floats * sizeof(float) + 255) & ~size_t(255));
}

hipError_t launch_decode_bf16(const Shape& s, int64_t pos, const void* q, const void* K,
                              const void* V, const void* Kd, const void* Vd, void* O, float* lse,
                              void* ws, hipStream_t st)
{
    const int64_t nseq = s.noncausal ? s.T : pos + 1;
    const DecodePlan pl = plan_decode(s, nseq);
    DecArgs a;
    a.q = (const uint16_t*)q;
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.Kd = (const uint16_t*)Kd;
    a.Vd = (const uint16_t*)Vd;
    a.O = (uint16_t*)O;
    a.lse = lse;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + (((size_t)pl.o_floats * sizeof(float) + 255) & ~size_t(255)));
    a.B = (int)s.B;
    a.Hq = (int)s.Hq;
    a.Hk = (int)s.Hk;
    a.T = (int)s.T;
    a.L = (int)s.L;
    a.G = s.G;
    a.W = s.L > 0 ? s.W : 0;
    a.pos = (int)pos;
    a.nseq = (int)nseq;
    a.nblk_seq = (int)pl.nblk_seq;
    a.nblk = (int)pl.nblk;
    a.nsplit = (int)pl.nsplit;
    a.c = s.scale * kLog2e;
    a.scale = s.scale;
    const dim3 grid1((unsigned)(s.B * s.Hk), (unsigned)pl.nsplit);   // nsplit <= 512
    const unsigned grid2 = (unsigned)(s.B * s.Hq * (s.d / 32));   // per query row and d-slice
    timing_begin("decode", st);
    if (s.d == 128)
        hipLaunchKernelGGL((decode_partial_kernel<128>), grid1, dim3(DEC_NW * 64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_partial_kernel<64>), grid1, dim3(DEC_NW * 64), 0, st, a);
    timing_end(st);
    timing_begin("decode_combine", st);
    if (s.d == 128)
        hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(grid2), dim3(COMB_WAVES * 64), 0, st, a);
    else
        hipLaunchKernelGGL((decode_combine_kernel<64>), dim3(grid2), dim3(COMB_WAVES * 64), 0, st, a);
    timing_end(st);
    return hipGetLastError();
}

}  // namespace moda
