// MoDA forward, bfloat16 storage, for gfx950.
//
// One workgroup owns one query chunk of one KV group: BM = 32*NW folded query
// rows i_q = t*G + g of batch b and KV head kv (the folded index and the
// grouped causal mask floor(i_q/G) >= i_k of "Mixture-of-Depths Attention",
// arXiv 2603.15619, paper summary, section 3.4 "The Unified Operator").  Each
// of the NW waves owns 32 consecutive folded rows, i.e. 32/G whole tokens with
// all G heads, as the 32 columns of its MFMA tiles.
//
// Sequence phase: K and V tiles of BN = 64 keys are staged in LDS (row-major,
// coalesced 16-byte loads, double-buffered) and shared by the NW waves and so
// by the G heads.  Per tile a wave computes S^T = K Q^T with 32x32x16 bf16 MFMA
// (fp32 accumulate), updates the online-softmax state (running max m, running
// sum, output accumulator o) with exp2, and accumulates O^T += V^T P^T with the
// V operand read transposed out of LDS (ds_read_b64_tr_b16).  Tiles entirely
// before the wave's first token skip the mask; later ones apply j <= t
// (the two sequence loops of the paper summary's "Hardware-Efficient
// Implementation", "Fused online-softmax (Algorithm 1)").
//
// Depth phase: each wave then reads only the depth rows of its own tokens,
// rows [t_lo*L, (t_hi+1)*L) of the token-major flattened depth KV, in blocks
// of 32 rows, masks with floor(r/L) == t (depth matching mask), and folds them
// into the same online-softmax state (group-aware depth loop of the same
// section).  The wave's columns hold all G heads of each token, so every depth
// row is fetched from HBM once and serves its G query rows through the MFMA.
//
// Epilogue: O = o / sum in bf16 (round to nearest even) and
// lse = scale*m + ln(sum) in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

struct FwdArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const uint16_t* Kd;
    const uint16_t* Vd;
    uint16_t* O;
    float* lse;
    int Hq, Hk, T, L, G;
    int nchunks;   // query chunks per (b, kv)
    float c;       // scale * log2(e)
    float scale;
};

constexpr int BN = 64;  // keys per sequence tile

// Sequence tiles beyond this threshold of max growth (log2 units) trigger a
// rescale of the running output and sum; below it the stale max is kept and the
// weights stay below 2^8, exactly representable in the same way.
constexpr float kRescaleLog2 = 8.f;

// Online-softmax update of one lane's column with the scores held in s[0..NB-1]
// (raw q.k values, 16 per block; masked entries are -inf).  The running max m
// is raised (and o, l rescaled by 2^(c(m - m_new))) only when some lane of the
// wave would otherwise see a weight above 2^kRescaleLog2; o/l = softmax output
// holds for any m, so keeping a stale m is exact.  On return s holds the
// weights exp2(c*(score - m)).
template <int D, int NB>
__device__ __forceinline__ void softmax_update(f32x16 (&s)[2], float& m, float& l,
                                               f32x16 (&o)[D / 32], float c)
{
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
    mt = max_halves(mt);
    const bool grow = (mt - m) * c > kRescaleLog2;   // true when m is still -inf
    if (__any(grow)) {
        const float m_new = fmaxf(m, mt);
        const float alpha = fast_exp2((m - m_new) * c);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        m = m_new;
    }
    const float mc = m * c;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = fast_exp2(fmaf(s[kb][j], c, -mc));
            s[kb][j] = p;
            ps += p;
        }
    l += sum_halves(ps);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void fwd_bf16_kernel(FwdArgs a)
{
    using TL = LdsTile<D>;
    constexpr int ELEMS = BN * TL::PITCH;      // one K or V tile
    static_assert(BN % (TL::RPI * NW) == 0, "tile staging must divide evenly");
    constexpr int BM = NW * 32;
    // [buf][K or V][BN rows]; the depth phase reuses it as NW private 32-row slices.
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * ELEMS];
    static_assert(NW * 32 * TL::PITCH <= 2 * 2 * ELEMS, "depth slices must fit");

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, hf = lane >> 5;
    const int G = a.G, T = a.T, L = a.L;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int unit = logical / a.nchunks;
    const int chunk = a.nchunks - 1 - logical % a.nchunks;   // heaviest chunks first
    const int b = unit / a.Hk, kv = unit % a.Hk;
    const int64_t TG = (int64_t)T * G;
    const int64_t r0 = (int64_t)chunk * BM;
    const int t_hi_wg = (int)min((r0 + BM - 1) / G, (int64_t)T - 1);

    const int64_t fw = r0 + 32 * w;              // first folded row of this wave
    const int64_t fcol = fw + col;               // this lane's column
    const bool valid = fcol < TG;
    const int tcol = (int)min(fcol / G, (int64_t)T - 1);
    const int hq = kv * G + (int)(fcol % G);
    const int tw_lo = (int)min(fw / G, (int64_t)T - 1);
    const int tw_hi = (int)min((fw + 31) / G, (int64_t)T - 1);

    const int64_t kvbase = ((int64_t)b * a.Hk + kv) * T;
    const uint16_t* Kb = a.K + kvbase * D;
    const uint16_t* Vb = a.V + kvbase * D;

    // Q^T columns as MFMA B operands: k-step si covers d = 16*si + 8*hf .. +8.
    bf16x8 qreg[D / 16];
    {
        const uint16_t* qrow = a.Q + (((int64_t)b * a.Hq + hq) * T + tcol) * D + 8 * hf;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) {
            uint4 v = valid ? ld16(qrow + 16 * si) : make_uint4(0, 0, 0, 0);
            qreg[si] = __builtin_bit_cast(bf16x8, v);
        }
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
    float m = -INFINITY, l = 0.f;

    // ---- sequence phase ----
    const int ntiles = t_hi_wg / BN + 1;
    // K and V tile `tile` into buffer `buf` (direct global->LDS; rows past T repeat row T-1,
    // whose weights are masked to zero).
    auto stage = [&](int tile, int buf) {
        uint16_t* ks = smem + (2 * buf) * ELEMS;
        const int k0 = tile * BN;
        stage_rows<D>(ks, BN, [&](int r) { return Kb + (int64_t)min(k0 + r, T - 1) * D; }, lane, w, NW);
        stage_rows<D>(ks + ELEMS, BN, [&](int r) { return Vb + (int64_t)min(k0 + r, T - 1) * D; },
                      lane, w, NW);
    };

    stage(0, 0);
    wait_vmem();
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntiles) stage(it + 1, buf ^ 1);
        const int k0 = it * BN;
        if (k0 <= tw_hi) {
            const uint16_t* ks = smem + (2 * buf) * ELEMS;
            const uint16_t* vs = ks + ELEMS;
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
#pragma unroll
                for (int si = 0; si < D / 16; ++si)
                    s[kb] = mfma32(lds_chunk<D>(ks, kb * 32 + col, 16 * si + 8 * hf), qreg[si], s[kb]);
            }
            if (k0 + BN - 1 > tw_lo) {   // tile reaches past the wave's first token: causal mask
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = k0 + kb * 32 + (j >> 2) * 8 + hf * 4 + (j & 3);
                        if (key > tcol) s[kb][j] = -INFINITY;
                    }
            }
            softmax_update<D, 2>(s, m, l, o, a.c);
            pv_block<D>(vs, 0, s[0], o, lane);
            pv_block<D>(vs, 32, s[1], o, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    // ---- depth phase: this wave's tokens only ----
    if (L > 0) {
        uint16_t* vslice = smem + w * 32 * TL::PITCH;   // private 32-row slice of the idle tiles
        const int64_t TL_rows = (int64_t)T * L;
        const uint16_t* Kdb = a.Kd + kvbase * (int64_t)L * D;
        const uint16_t* Vdb = a.Vd + kvbase * (int64_t)L * D;
        const int64_t dlo = (int64_t)tw_lo * L, dhi = (int64_t)(tw_hi + 1) * L;
        for (int64_t rb = dlo; rb < dhi; rb += 32) {
            // V rows of the block into the wave's slice; rows past the end are clamped.
            stage_rows<D>(vslice, 32, [&](int r) { return Vdb + min(rb + r, TL_rows - 1) * D; },
                          lane, 0, 1);
            // K rows as A operands straight from HBM.
            f32x16 s[2];
            {
                const int64_t r = min(rb + col, TL_rows - 1);
                const uint16_t* krow = Kdb + r * D + 8 * hf;
#pragma unroll
                for (int j = 0; j < 16; ++j) s[0][j] = 0.f;
#pragma unroll
                for (int si = 0; si < D / 16; ++si)
                    s[0] = mfma32(__builtin_bit_cast(bf16x8, ld16(krow + 16 * si)), qreg[si], s[0]);
            }
            // Row rb + (j/4)*8 + 4*hf + j%4 is visible iff it lies in [tcol*L, tcol*L + L).
            const int64_t lo = (int64_t)tcol * L - rb - 4 * hf;   // first visible row index
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rj = (j >> 2) * 8 + (j & 3);
                if (rj < lo || rj >= lo + L) s[0][j] = -INFINITY;
            }
            softmax_update<D, 1>(s, m, l, o, a.c);
            wait_vmem();
            wave_lds_sync();
            pv_block<D>(vslice, 0, s[0], o, lane);
            wave_lds_sync();
        }
    }

    // ---- epilogue ----
    if (valid) {
        const float inv = 1.f / l;
        uint16_t* orow = a.O + (((int64_t)b * a.Hq + hq) * T + tcol) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 v;
                v[0] = (__bf16)(o[db][4 * jj + 0] * inv);
                v[1] = (__bf16)(o[db][4 * jj + 1] * inv);
                v[2] = (__bf16)(o[db][4 * jj + 2] * inv);
                v[3] = (__bf16)(o[db][4 * jj + 3] * inv);
                *(bf16x4*)(orow + 32 * db + 8 * jj + 4 * hf) = v;
            }
        if (hf == 0) a.lse[((int64_t)b * a.Hq + hq) * T + tcol] = a.scale * m + __logf(l);
    }
}

template <int D, int NW>
hipError_t launch(const Shape& s, const FwdArgs& a, int nunits, hipStream_t st)
{
    const int64_t grid = (int64_t)nunits * a.nchunks;
    timing_begin("fwd", st);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
    timing_end(st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, void* O, float* lse, int rows_per_wg,
                           hipStream_t st)
{
    FwdArgs a;
    a.Q = (const uint16_t*)Q;
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.Kd = (const uint16_t*)Kd;
    a.Vd = (const uint16_t*)Vd;
    a.O = (uint16_t*)O;
    a.lse = lse;
    a.Hq = (int)s.Hq;
    a.Hk = (int)s.Hk;
    a.T = (int)s.T;
    a.L = (int)s.L;
    a.G = s.G;
    a.scale = s.scale;
    a.c = s.scale * kLog2e;
    const int64_t TG = s.T * s.G;
    a.nchunks = (int)((TG + rows_per_wg - 1) / rows_per_wg);
    const int nunits = (int)(s.B * s.Hk);
    if (s.d == 128) {
        return rows_per_wg == 256 ? launch<128, 8>(s, a, nunits, st)
                                  : launch<128, 4>(s, a, nunits, st);
    }
    return rows_per_wg == 256 ? launch<64, 8>(s, a, nunits, st) : launch<64, 4>(s, a, nunits, st);
}

}  // namespace moda
