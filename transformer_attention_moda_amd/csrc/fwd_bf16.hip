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
//
// Variants.  Non-causal (a runtime flag): every key 0..T-1 is visible, so every
// tile but a ragged last one skips the mask.  A depth window of the last W of L
// slots (a template instance of its own, so the full-depth kernel is unchanged):
// the depth phase gathers only the visible rows, W per token, into its 32-row
// blocks ("virtual rows" v -> token tw_lo + v / W, slot L - W + v % W), so it
// reads W/L of the depth bytes.
#include <type_traits>

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
    int W;         // visible depth slots per token (the last W of L)
    int noncausal; // every sequence key visible
    int scan;      // depth rows a wave scores: 0 its tokens', 1 its chunk's, 2 all (ablation)
    int nchunks;   // query chunks per (b, kv)
    float c;       // scale * log2(e)
    float scale;
};

constexpr int BN = 64;  // keys per sequence tile

// Adds the 8 bf16 values of p to acc (packed dot products with 1): the row sum of
// exactly the weights the PV product consumes, at half the instructions of fp32 adds.
__device__ __forceinline__ float row_sum_bf16(const bf16x8& p, float acc)
{
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[2 * i], p[2 * i + 1]}, one, acc, false);
    return acc;
}

// Eight waves per CU either way: one 8-wave workgroup (256 rows) or two 4-wave
// workgroups (128 rows), two waves per SIMD and at most 256 registers per wave.
template <int D, int NW, bool WIN>
__global__ __launch_bounds__(NW * 64, (D == 64 && NW == 4) ? 3 : 8 / NW) void fwd_bf16_kernel(FwdArgs a)
{
    using TL = LdsTile<D>;
    constexpr int ELEMS = BN * TL::PITCH;      // one K or V tile
    static_assert(BN % (TL::RPI * NW) == 0, "tile staging must divide evenly");
    constexpr int BM = NW * 32;
    // K and V tiles of buffers 0 and 1, one array each, so that the compiler can tell a
    // pending direct load into one buffer from reads of the other.  After the sequence
    // loop they hold the waves' private 32-row depth V slices, two per array; the depth K
    // slices go to ldk with 8 waves, and to the arrays the V slices leave free with 4.
    __shared__ __attribute__((aligned(16))) uint16_t lk0[ELEMS], lv0[ELEMS], lk1[ELEMS], lv1[ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t ldk[NW == 8 ? NW * 32 * D : 8];
    static_assert(ELEMS == 2 * 32 * TL::PITCH && (NW == 8 || NW == 4), "depth slices must fit");

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int lane_id = lane;
    const int col = lane & 31, hf = lane >> 5;
    const int G = a.G, T = a.T, L = a.L;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int unit = logical / a.nchunks;
    const int chunk = a.nchunks - 1 - logical % a.nchunks;   // heaviest chunks first
    const int b = unit / a.Hk, kv = unit % a.Hk;
    const int64_t TG = (int64_t)T * G;
    const int64_t r0 = (int64_t)chunk * BM;
    const bool nc = a.noncausal != 0;
    // Last key any query of the workgroup sees.
    const int t_hi_wg = nc ? T - 1 : (int)min((r0 + BM - 1) / G, (int64_t)T - 1);

    const int64_t fw = r0 + 32 * w;              // first folded row of this wave
    const int64_t fcol = fw + col;               // this lane's column
    const bool valid = fcol < TG;
    const int tcol = (int)min(fcol / G, (int64_t)T - 1);
    const int hq = kv * G + (int)(fcol % G);
    const int tw_lo = (int)min(fw / G, (int64_t)T - 1);
    const int tw_hi = (int)min((fw + 31) / G, (int64_t)T - 1);
    // Keys up to vis_lo are visible to every lane of the wave, keys up to vis_hi to some.
    const int vis_lo = nc ? T - 1 : tw_lo;
    const int vis_hi = nc ? T - 1 : tw_hi;

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
    // Running max: a finite sentinel, so that a block with no visible key for this lane
    // gives weights exp2(-inf) = 0, never NaN; the first visible score always triggers a
    // rescale (alpha = exp2(-huge) = 0).
    float m = -1e30f, l = 0.f;

    // ---- depth rows of this wave's tokens ----
    // The visible depth rows of tokens tw_lo..tw_hi, in blocks of 32: all of
    // [tw_lo*L, (tw_hi+1)*L) without a window; with one, W rows per token gathered as
    // virtual rows v (token tw_lo + v / W, slot L - W + v % W).  A block's K and V rows go
    // to the wave's two LDS slices by direct loads of 1 KiB contiguous rows per
    // instruction (loading K straight into registers as MFMA operands would request every
    // 128-byte line four times: 32 bytes of each of 32 rows per instruction).  Prefetch:
    // the next block's K loads are issued as soon as the current scores have read the K
    // slice, its V loads as soon as the current PV has read the V slice.  Mask: virtual
    // row v is visible to token t iff (t - tw_lo)*W <= v < (t - tw_lo)*W + W.
    auto depth_phase = [&]() {
        // Lane-derived values recomputed here from an opaque copy of the lane index, rather
        // than kept live (and spilled) across the sequence loop.
        const int lane = opaque(lane_id);
        const int hf = lane >> 5;
        const int tcol = (int)min((fw + (lane & 31)) / G, (int64_t)T - 1);
        const int64_t TL_rows = (int64_t)T * L;
        const uint16_t* Kdb = a.Kd + kvbase * (int64_t)L * D;
        const uint16_t* Vdb = a.Vd + kvbase * (int64_t)L * D;
        const int Wn = WIN ? a.W : L;
        // Tokens whose depth rows the wave scores: its own (the library's layout), or for
        // the ablation of the depth layouts its workgroup chunk's, or all T; the mask keeps
        // only the lane's own token, so the result is the same, the work is not.
        const int t_first = a.scan == 0 ? tw_lo : a.scan == 1 ? (int)min(r0 / G, (int64_t)T - 1) : 0;
        const int t_last = a.scan == 0 ? tw_hi
                         : a.scan == 1 ? (int)min((r0 + BM - 1) / G, (int64_t)T - 1) : T - 1;
        const int64_t dlo = (int64_t)t_first * L;
        const int64_t nv = (int64_t)(t_last - t_first + 1) * Wn;   // virtual rows of the wave
        const int nblk = (int)((nv + 31) / 32);
        // Depth row of virtual row v (v < nv).
        auto phys = [&](int64_t v) -> int64_t {
            if constexpr (!WIN) {
                return dlo + v;
            } else {
                const uint32_t vv = (uint32_t)v, tok = vv / (uint32_t)Wn;
                return (int64_t)(t_first + (int)tok) * L + (L - Wn) + (int)(vv - tok * (uint32_t)Wn);
            }
        };
        uint16_t* const arr = (w >> 1) == 0 ? lk0 : (w >> 1) == 1 ? lv0 : (w >> 1) == 2 ? lk1 : lv1;
        uint16_t* const vslot = arr + (w & 1) * 32 * D;
        uint16_t* const kslot = NW == 8 ? ldk + w * 32 * D : ((w >> 1) == 0 ? lk1 : lv1) + (w & 1) * 32 * D;
        constexpr int NI1 = 32 / TL::RPI;              // direct-load instructions per 32 rows
        // Rows past the wave's last visible row repeat a visible row (their weight is 0).
        auto issue = [&](int i, uint16_t* dst, const uint16_t* src) {
            const int64_t vb = 32 * (int64_t)i;
            if constexpr (!WIN) {
                const int64_t rb = dlo + vb;
                stage_rows<D>(dst, 32, src + rb * D,
                              [&](int r) { return (int)(min(rb + r, TL_rows - 1) - rb) * D; }, lane, 0, 1);
            } else {
                const int64_t rb = phys(vb);
                stage_rows<D>(dst, 32, src + rb * D,
                              [&](int r) { return (int)(phys(min(vb + r, nv - 1)) - rb) * D; }, lane, 0, 1);
            }
        };
        LaneOffsets<D> lof;
        lof.init(lane);
        if (nblk > 0) {
            issue(0, kslot, Kdb);
            issue(0, vslot, Vdb);
        }
        for (int i = 0; i < nblk; ++i) {
            const bool more = i + 1 < nblk;
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI1) : "memory");   // K of block i landed
            wave_lds_sync();
            f32x16 s[2];
#pragma unroll
            for (int j = 0; j < 16; ++j) s[0][j] = 0.f;
#pragma unroll
            for (int si = 0; si < D / 16; ++si)
                s[0] = mfma32(*(const bf16x8*)(kslot + lof.a[si]), qreg[si], s[0]);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");           // the K slice is read
            wave_lds_sync();
            if (more) issue(i + 1, kslot, Kdb);
            // first visible virtual row of this lane's token, relative to the lane's rows
            const int64_t lo = (int64_t)(tcol - t_first) * Wn - 32 * (int64_t)i - 4 * hf;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rj = (j >> 2) * 8 + (j & 3);
                if (rj < lo || rj >= lo + Wn) s[0][j] = -INFINITY;
            }
            softmax_update<D, 1>(s, m, l, o, a.c);
            if (more) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI1) : "memory");   // V of block i landed
            else wait_vmem();
            wave_lds_sync();
            pv_block<D>(vslot, 0, s[0], o, lane);
            wave_lds_sync();
            if (more) issue(i + 1, vslot, Vdb);
        }
    };

    // ---- sequence phase ----
    // Per-lane LDS element offsets, fixed for the whole loop (the tile base and
    // the 16-row-aligned block offsets below are compile-time immediates):
    //   kofs[si]     K operand of S^T = K Q^T, row col, chunk of d = 16*si + 8*hf;
    //   vofs[q][db]  transposed V read of pv_block, rows 8*q + 4*hf + (col%16)/4.
    int kofs[D / 16], vofs[2][D / 32];
#pragma unroll
    for (int si = 0; si < D / 16; ++si) kofs[si] = TL::off(col, 16 * si + 8 * hf);
    {
        const int krow = 4 * hf + ((col & 15) >> 2), dcol = 16 * (col >> 4) + 4 * (col & 3);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) vofs[q][db] = TL::off(krow + 8 * q, dcol + 32 * db);
    }
    // Direct-load staging: instruction i of this wave fills rows (w + i*NW)*RPI .. +RPI of a
    // tile; sofs[i] is this lane's element offset inside the global tile.
    constexpr int NI = BN / (TL::RPI * NW);
    int sofs[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = (w + i * NW) * TL::RPI + lane / TL::CPR;
        sofs[i] = r * D + ((lane % TL::CPR) ^ TL::swz(r)) * 8;
    }
    const int ntiles = t_hi_wg / BN + 1;
    // Last key every query of the workgroup sees: tiles wholly at or below it need no mask.
    const int t_lo_wg = nc ? T - 1 : (int)min(r0 / G, (int64_t)T - 1);
    const int n_full = (t_lo_wg + 1) / BN;     // tiles no wave of this workgroup needs to mask

    auto stage = [&](int tile, uint16_t* ks, uint16_t* vs) {
        const int k0 = tile * BN;
        if (k0 + BN <= T) {   // tile base as the scalar offset: k0*D*2 < 2^32 since T <= 2^24
            const uint32_t tb = (uint32_t)k0 * (2 * D);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int o = (w + i * NW) * TL::RPI * D;
                buffer_load_lds16(Kb, 2 * sofs[i], ks + o, tb);
                buffer_load_lds16(Vb, 2 * sofs[i], vs + o, tb);
            }
        } else {   // the sequence's last tile: rows past T repeat row T-1 (their weights are 0)
            const uint16_t* kt = Kb + (int64_t)k0 * D;
            const uint16_t* vt = Vb + (int64_t)k0 * D;
            auto rowofs = [&](int r) { return (min(k0 + r, T - 1) - k0) * D; };
            stage_rows<D>(ks, BN, kt, rowofs, lane, w, NW);
            stage_rows<D>(vs, BN, vt, rowofs, lane, w, NW);
        }
    };

    // One key tile from buffer BUF (0/1); MASKED tiles may reach past some wave's first token.
    auto step = [&](auto bufc, auto maskc, int it) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr bool MASKED = decltype(maskc)::value;
        const uint16_t* ks = BUF ? lk1 : lk0;
        const uint16_t* vs = BUF ? lv1 : lv0;
        if (it + 1 < ntiles) {
            if (BUF) stage(it + 1, lk0, lv0);
            else stage(it + 1, lk1, lv1);
        }
        const int k0 = it * BN;
        if (!MASKED || k0 <= vis_hi) {
            f32x16 s[2];
#pragma unroll
            for (int j = 0; j < 16; ++j) s[0][j] = s[1][j] = 0.f;
#pragma unroll
            for (int si = 0; si < D / 16; ++si) {
                const bf16x8 k0v = *(const bf16x8*)(ks + kofs[si]);
                const bf16x8 k1v = *(const bf16x8*)(ks + kofs[si] + 32 * D);
                s[0] = mfma32(k0v, qreg[si], s[0]);
                s[1] = mfma32(k1v, qreg[si], s[1]);
            }
            // K operand reads kept four ahead of the MFMAs that consume them.
            SCHED_GROUP(kSchedDsRead, 4);
#pragma unroll
            for (int i = 0; i < D / 8 - 4; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 1);
            }
            SCHED_GROUP(kSchedMfma, 4);
            if (MASKED && k0 + BN - 1 > vis_lo) {
                const int lim = nc ? T - 1 : tcol;   // last key this lane sees
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = k0 + kb * 32 + (j >> 2) * 8 + hf * 4 + (j & 3);
                        if (key > lim) s[kb][j] = -INFINITY;
                    }
            }
            softmax_update<D, 2, false>(s, m, l, o, a.c);
            float ps = 0.f;   // row sum of this tile's weights, as rounded for the PV product
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    const f32x16& p = s[kb];
                    const bf16x8 pb = to_bf16x8(p[8 * sp + 0], p[8 * sp + 1], p[8 * sp + 2],
                                                p[8 * sp + 3], p[8 * sp + 4], p[8 * sp + 5],
                                                p[8 * sp + 6], p[8 * sp + 7]);
                    ps = row_sum_bf16(pb, ps);
                    const int rowoff = (kb * 32 + 16 * sp) * D;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const bf16x4 lo = lds_read_tr(vs + vofs[0][db] + rowoff);
                        const bf16x4 hi = lds_read_tr(vs + vofs[1][db] + rowoff);
                        const bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        o[db] = mfma32(av, pb, o[db]);
                    }
                }
            l += sum_halves(ps);
        }
        wait_vmem();
        __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BF = std::integral_constant<bool, false>;
    using BT = std::integral_constant<bool, true>;
    stage(0, lk0, lv0);
    wait_vmem();
    __syncthreads();
    int it = 0;
    for (; it + 1 < n_full; it += 2) {
        step(I0(), BF(), it);
        step(I1(), BF(), it + 1);
    }
    for (; it < ntiles; ++it) {
        if (it < n_full) {
            if (it & 1) step(I1(), BF(), it);
            else step(I0(), BF(), it);
        } else {
            if (it & 1) step(I1(), BT(), it);
            else step(I0(), BT(), it);
        }
    }
    if (L > 0) depth_phase();

    // ---- epilogue ----
    {   // lane-derived values recomputed, as in the depth phase
        const int lane = opaque(lane_id);
        const int hf = lane >> 5;
        const int64_t fcol = fw + (lane & 31);
        const int tcol = (int)min(fcol / G, (int64_t)T - 1);
        const int hq = kv * G + (int)(fcol % G);
        if (fcol < TG) {
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
}

template <int D, int NW>
hipError_t launch(const Shape& s, const FwdArgs& a, int nunits, hipStream_t st)
{
    const int64_t grid = (int64_t)nunits * a.nchunks;
    timing_begin("fwd", st);
    if (a.L > 0 && a.W < a.L)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, true>), dim3((unsigned)grid), dim3(NW * 64), 0,
                           st, a);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, false>), dim3((unsigned)grid), dim3(NW * 64), 0,
                           st, a);
    timing_end(st);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, void* O, float* lse, int rows_per_wg,
                           hipStream_t st, int scan)
{
    FwdArgs a;
    a.scan = scan;
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
    a.W = s.W;
    a.noncausal = s.noncausal ? 1 : 0;
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
