// MoDA backward, bfloat16 storage, for gfx950.
//
// The gradients of the operator of "Mixture-of-Depths Attention" (arXiv
// 2603.15619, paper summary, section 3.4: one softmax over the causal
// sequence keys and the token's own L depth keys).  With p the softmax weights
// (recomputed from the forward's log-sum-exp), D = <dO, O> and
// dS = p (dO.v - D) for every visible key/value pair (v in V or V_depth):
//   dQ  = scale (sum over sequence keys of dS K + sum over own depth rows of dS Kd)
//   dK  = scale sum over queries of dS Q,      dV  = sum over queries of p dO
//   dKd = scale sum over the token's G heads of dS Q, dVd = same with p dO
//
// Four kernels, none with atomics (results are deterministic); bwd_dkdv depends only
// on bwd_pre, the other two run in this order:
//   bwd_pre    D and lse in log2 units, one per query row (workspace);
//   bwd_depth  per wave, its tokens' depth rows: S_d = Q Kd^T (lane = depth
//              row), dVd^T += dO^T P_d, dKd^T += Q^T dS_d, and the depth part of
//              dQ^T += Kd^T dS_d^T (fp32 rows in the workspace).  A token's G
//              heads sit in one wave, so every depth row is finished by one wave;
//   bwd_dq     query-stationary like the forward: per key tile S^T = K Q^T,
//              dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T with K read
//              transposed from LDS; adds the depth part and stores dQ;
//   bwd_dkdv   key-stationary: each wave keeps 32 keys of K and V as MFMA
//              operands and walks the query rows that see them:
//              S = Q K^T, dP = dO V^T (lane = key), dV^T += dO^T P and
//              dK^T += Q^T dS with dO and Q read transposed from LDS.
//
// Streams.  On small problems (at most 1024 key workgroups of 4 waves) the key-stationary
// pass runs on a second stream of the device, forked from the caller's stream after
// bwd_pre by an event and joined back into it by another, so that it shares the chip with
// bwd_depth and bwd_dq: each kernel's last, partly idle stretch is filled by the other.
// On larger grids the tails are a small part of the time and the two kernels on one chip
// slow each other, so they run one after the other on the caller's stream.
//
// Variants.  Non-causal (runtime flag): every key is visible to every query, so
// bwd_dq walks all key tiles and bwd_dkdv all query rows, masking only ragged
// ends.  A depth window (the last W of L slots): bwd_depth gives the hidden
// slots weight 0, so their dKd, dVd rows are written as exact zeros and they add
// nothing to dQ.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

struct BwdArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const uint16_t* Kd;
    const uint16_t* Vd;
    const uint16_t* O;
    const float* lse;
    const uint16_t* dO;
    uint16_t* dQ;
    uint16_t* dK;
    uint16_t* dV;
    uint16_t* dKd;
    uint16_t* dVd;
    float* lse2;   // lse * log2(e), [B*Hq*T]
    float* Dv;     // <dO, O>,        [B*Hq*T]
    float* dqd;    // depth part of dQ / scale, fp32 [B*Hq*T][d] (L > 0)
    int Hq, Hk, T, L, G, lgG;
    int W;         // visible depth slots per token (the last W of L)
    int noncausal; // every sequence key visible
    int nblocks;   // work blocks per (b, kv) of the launched kernel
    float c;       // scale * log2(e)
    float scale;
    int64_t rows;  // B*Hq*T
    float* part;       // bwd_dkdv split: fp32 partial dK, dV per piece [grid][2][128][d]
    int piece_tiles;   // bwd_dkdv: query tiles per piece of a split key block (0: no split)
    int nkeyblocks;    // bwd_dkdv: key blocks per (b, kv)
};

constexpr int BN = 64;  // sequence keys per tile (bwd_dq)

// ---------------------------------------------------------------- bwd_pre
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a)
{
    constexpr int LPR = D / 8;            // lanes per row (16 bytes each)
    constexpr int RPB = 256 / LPR;        // rows per block
    const int sub = threadIdx.x % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const bool ok = row < a.rows;
    float acc = 0.f;
    if (ok) {
        const uint4 x = ld16(a.dO + row * D + sub * 8);
        const uint4 y = ld16(a.O + row * D + sub * 8);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc += __uint_as_float(xs[i] << 16) * __uint_as_float(ys[i] << 16);
            acc += __uint_as_float(xs[i] & 0xffff0000u) * __uint_as_float(ys[i] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (ok && sub == 0) {
        a.Dv[row] = acc;
        a.lse2[row] = a.lse[row] * kLog2e;
    }
}

// ---------------------------------------------------------------- bwd_dq
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, D == 64 ? 3 : 1) void bwd_dq_kernel(BwdArgs a)
{
    using TL = LdsTile<D>;
    constexpr int ELEMS = BN * TL::PITCH;
    static_assert(BN % (TL::RPI * NW) == 0, "tile staging must divide evenly");
    constexpr int BM = NW * 32;
    // Per buffer: the K tile, then the V tile.  One array for both buffers: apart, the
    // compiler keeps more operand addresses live and this kernel spills (8 registers, about
    // 4% slower).  The price of one array: the compiler waits for the next tile's load
    // before the transposed K reads of the dQ product, by when it has mostly landed.
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * ELEMS];
    uint16_t* const lb0 = smem;
    uint16_t* const lb1 = smem + 2 * ELEMS;

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int col = lane & 31, hf = lane >> 5;
    const int G = a.G, T = a.T, L = a.L;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int unit = logical / a.nblocks;
    const int chunk = a.nblocks - 1 - logical % a.nblocks;
    const int b = unit / a.Hk, kv = unit % a.Hk;
    const int64_t TG = (int64_t)T * G;
    const int64_t r0 = (int64_t)chunk * BM;
    const bool nc = a.noncausal != 0;
    const int t_hi_wg = nc ? T - 1 : (int)min((r0 + BM - 1) / G, (int64_t)T - 1);
    const int64_t fw = r0 + 32 * w, fcol = fw + col;
    const bool valid = fcol < TG;
    const int tcol = (int)min(fcol / G, (int64_t)T - 1);
    const int hq = kv * G + (int)(fcol % G);
    // Keys up to vis_lo are visible to every lane of the wave, keys up to vis_hi to some.
    const int vis_lo = nc ? T - 1 : (int)min(fw / G, (int64_t)T - 1);
    const int vis_hi = nc ? T - 1 : (int)min((fw + 31) / G, (int64_t)T - 1);

    const int64_t kvbase = ((int64_t)b * a.Hk + kv) * T;
    const uint16_t* Kb = a.K + kvbase * D;
    const uint16_t* Vb = a.V + kvbase * D;
    const int64_t qrow_idx = ((int64_t)b * a.Hq + hq) * T + tcol;

    bf16x8 qreg[D / 16], dreg[D / 16];
    {
        const uint16_t* qrow = a.Q + qrow_idx * D + 8 * hf;
        const uint16_t* drow = a.dO + qrow_idx * D + 8 * hf;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) {
            qreg[si] = __builtin_bit_cast(bf16x8, valid ? ld16(qrow + 16 * si) : make_uint4(0, 0, 0, 0));
            dreg[si] = __builtin_bit_cast(bf16x8, valid ? ld16(drow + 16 * si) : make_uint4(0, 0, 0, 0));
        }
    }
    const float lse2 = valid ? a.lse2[qrow_idx] : INFINITY;
    const float Dr = valid ? a.Dv[qrow_idx] : 0.f;
    const float c = a.c;

    f32x16 dq[D / 32];
    zero(dq);

    LaneOffsets<D> lo;
    lo.init(lane);
    constexpr int NI = BN / (TL::RPI * NW);
    int sofs[NI];
#pragma unroll
    for (int i2 = 0; i2 < NI; ++i2) {
        const int r = (w + i2 * NW) * TL::RPI + lane / TL::CPR;
        sofs[i2] = r * D + ((lane % TL::CPR) ^ TL::swz(r)) * 8;
    }
    const int ntiles = t_hi_wg / BN + 1;
    const int t_lo_wg = nc ? T - 1 : (int)min(r0 / G, (int64_t)T - 1);
    const int n_full = (t_lo_wg + 1) / BN;     // tiles no wave of this workgroup needs to mask
    auto stage = [&](int tile, uint16_t* ks) {
        uint16_t* const vs = ks + ELEMS;
        const int k0 = tile * BN;
        const uint16_t* kt = Kb + (int64_t)k0 * D;
        const uint16_t* vt = Vb + (int64_t)k0 * D;
        if (k0 + BN <= T) {
#pragma unroll
            for (int i2 = 0; i2 < NI; ++i2) {
                const int o = (w + i2 * NW) * TL::RPI * D;
                buffer_load_lds16(kt, 2 * sofs[i2], ks + o);
                buffer_load_lds16(vt, 2 * sofs[i2], vs + o);
            }
        } else {   // the sequence's last tile: rows past T repeat row T-1 (their weights are 0)
            auto rowofs = [&](int r) { return (min(k0 + r, T - 1) - k0) * D; };
            stage_rows<D>(ks, BN, kt, rowofs, lane, w, NW);
            stage_rows<D>(vs, BN, vt, rowofs, lane, w, NW);
        }
    };
    auto step = [&](auto bufc, auto maskc, int it) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr bool MASKED = decltype(maskc)::value;
        const uint16_t* ks = BUF ? lb1 : lb0;
        const uint16_t* vs = ks + ELEMS;
        if (it + 1 < ntiles) stage(it + 1, BUF ? lb0 : lb1);
        const int k0 = it * BN;
        if (!MASKED || k0 <= vis_hi) {
            f32x16 sv[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) sv[kb][j] = dp[kb][j] = 0.f;
#pragma unroll
                for (int si = 0; si < D / 16; ++si) {
                    sv[kb] = mfma32(*(const bf16x8*)(ks + lo.a[si] + kb * 32 * D), qreg[si], sv[kb]);
                    dp[kb] = mfma32(*(const bf16x8*)(vs + lo.a[si] + kb * 32 * D), dreg[si], dp[kb]);
                }
            }
            // K and V operand reads kept 4 ahead of the score MFMAs.
            SCHED_GROUP(kSchedDsRead, 4);
#pragma unroll
            for (int i = 0; i < 2 * D / 8 - 4; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 1);
            }
            SCHED_GROUP(kSchedMfma, 4);
            const bool need_mask = MASKED && k0 + BN - 1 > vis_lo;
            const int lim = nc ? T - 1 : tcol;   // last key this lane sees
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float pr = fast_exp2(fmaf(sv[kb][j], c, -lse2));
                    if (MASKED) {
                        const int key = k0 + kb * 32 + (j >> 2) * 8 + hf * 4 + (j & 3);
                        if (need_mask && key > lim) pr = 0.f;
                    }
                    sv[kb][j] = pr * (dp[kb][j] - Dr);
                }
            pv_block_pre<D>(ks, sv[0], dq, lo);
            pv_block_pre<D>(ks + 32 * D, sv[1], dq, lo);
            // Transposed K reads of the dQ product kept 4 MFMAs ahead.
            SCHED_GROUP(kSchedDsRead, 8);
#pragma unroll
            for (int i = 0; i < 2 * D / 16 - 4; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 2);
            }
            SCHED_GROUP(kSchedMfma, 4);
        }
        wait_vmem();
        __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BF = std::integral_constant<bool, false>;
    using BT = std::integral_constant<bool, true>;
    stage(0, lb0);
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

    // The depth rows' part (bwd_depth ran before this kernel).
    if (L > 0 && valid) {
        const float* drow = a.dqd + qrow_idx * D + 4 * hf;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float4 v = *(const float4*)(drow + 32 * db + 8 * jj);
                dq[db][4 * jj + 0] += v.x;
                dq[db][4 * jj + 1] += v.y;
                dq[db][4 * jj + 2] += v.z;
                dq[db][4 * jj + 3] += v.w;
            }
    }
    if (valid) store_row_bf16<D>(a.dQ + qrow_idx * D, dq, a.scale, lane);
}

// ---------------------------------------------------------------- bwd_dkdv
constexpr int BQ = 64;  // folded query rows per staged tile (bwd_dkdv)

// WPS: waves per SIMD the registers are budgeted for.  At d = 128 the accumulators and
// operands need about 480 registers: one.  At d = 64 two fit in 256 registers each (a few
// spills outside the tile loop's main path) and the second wave hides LDS latency, 10-15%
// faster once there are enough workgroups (launched as 8-wave workgroups of 256 keys); on
// small grids, where every workgroup is resident at once and the heaviest key block sets
// the time, one wave with the whole register file is faster.
// SPLIT: the launch splits key blocks' query walks into pieces (small grids); a separate
// instance, so that the unsplit kernels carry none of its code.
template <int D, int NW, int WPS, bool SPLIT>
__global__ __launch_bounds__(NW * 64, WPS) void bwd_dkdv_kernel(BwdArgs a)
{
    using TL = LdsTile<D>;
    static_assert(BQ % (TL::RPI * NW) == 0, "tile staging must divide evenly");
    constexpr int BK = NW * 32;   // keys per workgroup
    constexpr int TILE = BQ * D;  // elements of one Q or dO tile
    // Per buffer: the Q and dO tiles, then the tiles' lse2 and D rows.  One array per
    // buffer, so that the compiler can tell a pending load into one buffer from reads of
    // the other (and keeps a single address register per operand for both tiles).
    __shared__ __attribute__((aligned(16))) uint16_t lb0[2 * TILE], lb1[2 * TILE];
    __shared__ __attribute__((aligned(16))) float sr0[2 * BQ], sr1[2 * BQ];

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int col = lane & 31, hf = lane >> 5;
    const int G = a.G, T = a.T, lgG = a.lgG;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int unit = logical / a.nblocks;
    int kblk = logical % a.nblocks;   // small key blocks see the most queries: first
    // Split walks (small grids): work block r of a unit is piece r - (pieces of the key
    // blocks before it) of the first key block whose pieces reach past r.
    int piece = 0, npieces = 1;
    if constexpr (SPLIT) {
        const int64_t TGs = (int64_t)T * G;
        const bool ncs = a.noncausal != 0;
        // Query tiles key block k walks: from the first folded row that sees one of its keys.
        auto tiles_of = [&](int k) {
            return (int)((TGs - (ncs ? 0 : (int64_t)k * BK * G) + BQ - 1) / BQ);
        };
        int r = kblk;
        for (kblk = 0;; ++kblk) {
            const int n = (tiles_of(kblk) + a.piece_tiles - 1) / a.piece_tiles;
            if (r < n) {
                npieces = n;
                piece = r;
                break;
            }
            r -= n;
        }
    }
    const int b = unit / a.Hk, kv = unit % a.Hk;
    const int k0 = kblk * BK, kw = k0 + 32 * w, key = kw + col;
    const bool kvalid = key < T;
    const int64_t kvbase = ((int64_t)b * a.Hk + kv) * T;

    bf16x8 kreg[D / 16], vreg[D / 16];
    {
        const uint16_t* krow = a.K + (kvbase + key) * D + 8 * hf;
        const uint16_t* vrow = a.V + (kvbase + key) * D + 8 * hf;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) {
            kreg[si] = __builtin_bit_cast(bf16x8, kvalid ? ld16(krow + 16 * si) : make_uint4(0, 0, 0, 0));
            vreg[si] = __builtin_bit_cast(bf16x8, kvalid ? ld16(vrow + 16 * si) : make_uint4(0, 0, 0, 0));
        }
    }
    f32x16 dk[D / 32], dv[D / 32];
    zero(dk);
    zero(dv);
    LaneOffsets<D> lo;
    lo.init(lane);

    const int64_t TG = (int64_t)T * G;
    const bool nc = a.noncausal != 0;
    // First folded row that sees a key of this block, and the leading tiles that hold rows
    // not seeing some key of it (causal only: non-causal rows see every key).
    const int64_t f_start = nc ? 0 : (int64_t)k0 * G;
    const int ntiles = (int)((TG - f_start + BQ - 1) / BQ);
    const int n_mask = nc ? 0 : min(ntiles, ((BK - 1) * G + BQ - 1) / BQ);
    // This work block's tiles [it_begin, it_end) of the walk.
    const int it_begin = SPLIT ? piece * a.piece_tiles : 0;
    const int it_end = SPLIT && npieces > 1 ? min(ntiles, it_begin + a.piece_tiles) : ntiles;
    const int64_t qhead0 = (int64_t)b * a.Hq + (int64_t)kv * G;

    // Folded row f0 + r (f0 a multiple of BQ, G | BQ) is query head qhead0 + r%G at token
    // f0/G + r/G: a uniform base plus a per-lane constant.
    constexpr int NI = BQ / (TL::RPI * NW);
    int sofs[NI];
#pragma unroll
    for (int i2 = 0; i2 < NI; ++i2) {
        const int r = (w + i2 * NW) * TL::RPI + lane / TL::CPR;
        sofs[i2] = (int)(((int64_t)(r & (G - 1)) * T + (r >> lgG)) * D) +
                   ((lane % TL::CPR) ^ TL::swz(r)) * 8;
    }
    static_assert(BQ == 64, "one wave stages a tile's lse2 and D rows");
    const uint32_t rofs = 4u * (uint32_t)((lane & (G - 1)) * T + (lane >> lgG));   // lse/D byte offset
    auto qi_of = [&](int64_t f) {
        f = min(f, TG - 1);
        return (qhead0 + (f & (G - 1))) * T + (f >> lgG);
    };
    auto stage = [&](int tile, uint16_t* qs, float* sr) {
        uint16_t* const ds = qs + TILE;
        const int64_t f0 = f_start + (int64_t)tile * BQ;
        const int64_t base = qhead0 * T + (f0 >> lgG);   // row of folded row f0 (f0 % G == 0)
        const uint16_t* qt = a.Q + base * D;
        const uint16_t* dt = a.dO + base * D;
        if (f0 + BQ <= TG) {
#pragma unroll
            for (int i2 = 0; i2 < NI; ++i2) {
                const int o = (w + i2 * NW) * TL::RPI * D;
                buffer_load_lds16(qt, 2 * sofs[i2], qs + o);
                buffer_load_lds16(dt, 2 * sofs[i2], ds + o);
            }
            if (w == 0) {
                buffer_load_lds<4>(a.lse2 + base, rofs, sr);
                buffer_load_lds<4>(a.Dv + base, rofs, sr + BQ);
            }
        } else {   // the last tile: rows past the end repeat the last row with lse +inf (weight 0)
            auto rowofs = [&](int r) { return (int)(qi_of(f0 + r) - base) * D; };
            stage_rows<D>(qs, BQ, qt, rowofs, lane, w, NW);
            stage_rows<D>(ds, BQ, dt, rowofs, lane, w, NW);
            if (w == 0) {
                const int64_t f = f0 + lane;
                sr[lane] = f < TG ? a.lse2[qi_of(f)] : INFINITY;
                sr[BQ + lane] = f < TG ? a.Dv[qi_of(f)] : 0.f;
            }
        }
    };

    const float c = a.c;
    auto step = [&](auto bufc, auto maskc, int it) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr bool MASKED = decltype(maskc)::value;
        const uint16_t* qs = BUF ? lb1 : lb0;
        const uint16_t* ds = qs + TILE;
        const float* sr = BUF ? sr1 : sr0;
        if (it + 1 < it_end) {
            if (BUF) stage(it + 1, lb0, sr0);
            else stage(it + 1, lb1, sr1);
        }
        const int64_t f0 = f_start + (int64_t)it * BQ;
        // Weights of block qb: P = exp2(S c - lse2) (masked), dS = P (dP - D).
        auto weights = [&](int qb, f32x16& sv, f32x16& dp) {
            // 32-bit folded row (T*G < 2^31): 64-bit row constants of the mask would be
            // hoisted out of the loop and spilled.
            const int fb = (int)f0 + qb * 32;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rbase = qb * 32 + jj * 8 + 4 * hf;
                const float4 l4 = *(const float4*)&sr[rbase];
                const float4 d4 = *(const float4*)&sr[BQ + rbase];
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * jj + e;
                    float pr = fast_exp2(fmaf(sv[j], c, -lv[e]));
                    if (MASKED && ((fb + jj * 8 + 4 * hf + e) >> lgG) < key) pr = 0.f;
                    sv[j] = pr;
                    dp[j] = pr * (dp[j] - dvv[e]);
                }
            }
        };
        if (MASKED) {
#pragma unroll
            for (int qb = 0; qb < BQ / 32; ++qb) {
                const int64_t fb = f0 + qb * 32;
                if (((fb + 31) >> lgG) < kw || fb >= TG) continue;   // nothing visible
                f32x16 sv, dp;
#pragma unroll
                for (int j = 0; j < 16; ++j) sv[j] = dp[j] = 0.f;
#pragma unroll
                for (int si = 0; si < D / 16; ++si) {
                    sv = mfma32(*(const bf16x8*)(qs + lo.a[si] + qb * 32 * D), kreg[si], sv);
                    dp = mfma32(*(const bf16x8*)(ds + lo.a[si] + qb * 32 * D), vreg[si], dp);
                }
                weights(qb, sv, dp);
                pv_block_pre<D>(ds + qb * 32 * D, sv, dv, lo);
                pv_block_pre<D>(qs + qb * 32 * D, dp, dk, lo);
            }
        } else {
            // Both blocks' scores first, so that block 0's weights overlap block 1's
            // products and block 1's weights overlap block 0's gradient products.
            f32x16 sv[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) sv[qb][j] = dp[qb][j] = 0.f;
#pragma unroll
                for (int si = 0; si < D / 16; ++si) {
                    sv[qb] = mfma32(*(const bf16x8*)(qs + lo.a[si] + qb * 32 * D), kreg[si], sv[qb]);
                    dp[qb] = mfma32(*(const bf16x8*)(ds + lo.a[si] + qb * 32 * D), vreg[si], dp[qb]);
                }
            }
            weights(0, sv[0], dp[0]);
            pv_block_pre<D>(ds, sv[0], dv, lo);
            pv_block_pre<D>(qs, dp[0], dk, lo);
            weights(1, sv[1], dp[1]);
            pv_block_pre<D>(ds + 32 * D, sv[1], dv, lo);
            pv_block_pre<D>(qs + 32 * D, dp[1], dk, lo);
            // Issue order (one wave per SIMD, so nothing else hides LDS latency): LA
            // operand reads ahead of the score MFMAs, GA read pairs of the gradient
            // products issued during the last score MFMAs, and each block's weight
            // arithmetic spread over MFMAs that do not depend on it.
            constexpr int NM = D / 8;   // score MFMAs per block (S and dP)
            constexpr int NG = D / 8;   // gradient MFMAs per block (dV and dK)
            constexpr int LA = 16, GA = 16;
            SCHED_GROUP(kSchedDsRead, LA);
#pragma unroll
            for (int i = 0; i < 2 * NM - LA; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 1);
                if (i >= NM) SCHED_GROUP(kSchedValu, 5);
            }
#pragma unroll
            for (int i = 0; i < LA; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 2 * GA / LA);
                SCHED_GROUP(kSchedValu, 5);
            }
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 2);
                SCHED_GROUP(kSchedValu, 5);
            }
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                SCHED_GROUP(kSchedMfma, 1);
                SCHED_GROUP(kSchedDsRead, 2);
            }
        }
        wait_vmem();
        __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BF = std::integral_constant<bool, false>;
    using BT = std::integral_constant<bool, true>;
    // Tile it is staged into buffer it & 1.
    if (it_begin < it_end) {
        if (it_begin & 1) stage(it_begin, lb1, sr1);
        else stage(it_begin, lb0, sr0);
    }
    wait_vmem();
    __syncthreads();
    int it = it_begin;
    for (; it < (SPLIT ? min(n_mask, it_end) : n_mask); ++it) {
        if (it & 1) step(I1(), BT(), it);
        else step(I0(), BT(), it);
    }
    if (it < it_end && (it & 1)) {
        step(I1(), BF(), it);
        ++it;
    }
    for (; it + 1 < it_end; it += 2) {
        step(I0(), BF(), it);
        step(I1(), BF(), it + 1);
    }
    if (it < it_end) step(I0(), BF(), it);
    if (kvalid) {
        if (!SPLIT || npieces == 1) {
            store_row_bf16<D>(a.dK + (kvbase + key) * D, dk, a.scale, lane);
            store_row_bf16<D>(a.dV + (kvbase + key) * D, dv, 1.f, lane);
        } else {   // partial sums of this piece, unscaled; dkdv_reduce_kernel adds the pieces
            float* pk = a.part + ((int64_t)logical * 2 * BK + (key - k0)) * D;
            store_row_f32<D>(pk, dk, lane);
            store_row_f32<D>(pk + (int64_t)BK * D, dv, lane);
        }
    }
}

// Split key blocks (bwd_dkdv with piece_tiles > 0): dK, dV of each key block walked in
// more than one piece are the sum of its pieces' partials, added in piece order (so the
// result does not depend on scheduling).  One workgroup per (b, kv, key block).
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(BwdArgs a)
{
    constexpr int BK = 128;
    const int unit = blockIdx.x / a.nkeyblocks, kblk = blockIdx.x % a.nkeyblocks;
    const int64_t TG = (int64_t)a.T * a.G;
    const bool nc = a.noncausal != 0;
    int first = 0, np = 0;
    for (int k = 0; k <= kblk; ++k) {
        const int nt = (int)((TG - (nc ? 0 : (int64_t)k * BK * a.G) + BQ - 1) / BQ);
        const int n = (nt + a.piece_tiles - 1) / a.piece_tiles;
        if (k == kblk) np = n;
        else first += n;
    }
    if (np <= 1) return;   // written directly by its one piece
    const int b = unit / a.Hk, kv = unit % a.Hk;
    const int k0 = kblk * BK;
    const int64_t kvbase = ((int64_t)b * a.Hk + kv) * a.T;
    const float* p0 = a.part + ((int64_t)unit * a.nblocks + first) * 2 * BK * D;
    for (int e = 4 * threadIdx.x; e < BK * D; e += 4 * 256) {
        const int key = k0 + e / D;
        if (key >= a.T) break;
        float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
        for (int p = 0; p < np; ++p) {
            const float4 vk = *(const float4*)(p0 + (int64_t)p * 2 * BK * D + e);
            const float4 vv = *(const float4*)(p0 + (int64_t)p * 2 * BK * D + BK * D + e);
            sk.x += vk.x; sk.y += vk.y; sk.z += vk.z; sk.w += vk.w;
            sv.x += vv.x; sv.y += vv.y; sv.z += vv.z; sv.w += vv.w;
        }
        const bf16x4 ok = {(__bf16)(sk.x * a.scale), (__bf16)(sk.y * a.scale), (__bf16)(sk.z * a.scale),
                           (__bf16)(sk.w * a.scale)};
        const bf16x4 ov = {(__bf16)sv.x, (__bf16)sv.y, (__bf16)sv.z, (__bf16)sv.w};
        *(bf16x4*)(a.dK + (kvbase + key) * D + e % D) = ok;
        *(bf16x4*)(a.dV + (kvbase + key) * D + e % D) = ov;
    }
}

// ---------------------------------------------------------------- bwd_depth
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, D == 64 ? 2 : 1) void bwd_depth_kernel(BwdArgs a)
{
    using TL = LdsTile<D>;
    constexpr int BM = NW * 32;
    __shared__ __attribute__((aligned(16))) uint16_t smem[NW][2][32 * TL::PITCH];   // per wave: Q, dO rows
    // per wave: the depth block's Kd rows for the transposed read, then its output rows
    __shared__ __attribute__((aligned(16))) uint16_t sout[NW][32 * TL::PITCH];
    constexpr int TP = 36;   // dS_d^T rows (depth rows x 32 queries), padded against bank conflicts
    __shared__ __attribute__((aligned(16))) uint16_t sds[NW][32 * TP];
    __shared__ __attribute__((aligned(16))) float srow[NW][2][32];            // per wave: lse2, D

    const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
    const int col = lane & 31, hf = lane >> 5;
    const int G = a.G, T = a.T, L = a.L, lgG = a.lgG;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int unit = logical / a.nblocks;
    const int chunk = logical % a.nblocks;
    const int b = unit / a.Hk, kv = unit % a.Hk;
    const int64_t TG = (int64_t)T * G;
    const int64_t fw = (int64_t)chunk * BM + 32 * w;
    if (fw >= TG) return;   // wave-uniform; no workgroup barrier below
    const int tw_lo = (int)(fw >> lgG);
    const int tw_hi = (int)min((fw + 31) >> lgG, (int64_t)T - 1);
    const int64_t qhead0 = (int64_t)b * a.Hq + (int64_t)kv * G;
    const int64_t kvbase = ((int64_t)b * a.Hk + kv) * T;

    uint16_t* qs = smem[w][0];
    uint16_t* ds = smem[w][1];
    // This wave's 32 query rows (folded) into its slices; rows past the end repeat the last
    // row, and their lse of +inf gives them zero weight.
    auto qi_of = [&](int64_t f) {
        f = min(f, TG - 1);
        return (qhead0 + (f & (G - 1))) * T + (f >> lgG);
    };
    {
        const int64_t q0 = qi_of(fw);   // fw % G == 0, so later rows sit at or after it
        auto rowofs = [&](int r) { return (int)(qi_of(fw + r) - q0) * D; };
        stage_rows<D>(qs, 32, a.Q + q0 * D, rowofs, lane, 0, 1);
        stage_rows<D>(ds, 32, a.dO + q0 * D, rowofs, lane, 0, 1);
    }
    if (lane < 32) {
        const int64_t f = fw + lane;
        float lv = INFINITY, dvv = 0.f;
        if (f < TG) {
            const int64_t qi = (qhead0 + (f & (G - 1))) * T + (f >> lgG);
            lv = a.lse2[qi];
            dvv = a.Dv[qi];
        }
        srow[w][0][lane] = lv;
        srow[w][1][lane] = dvv;
    }
    wait_vmem();
    wave_lds_sync();
    // Query rows as MFMA A operands (lane row l%32, k = d 16*si + 8*hf .. +8), read from
    // the slices for every block.
    LaneOffsets<D> lo;
    lo.init(lane);

    const float c = a.c;
    const int64_t TL_rows = (int64_t)T * L;
    const uint16_t* Kdb = a.Kd + kvbase * (int64_t)L * D;
    const uint16_t* Vdb = a.Vd + kvbase * (int64_t)L * D;
    uint16_t* dKdb = a.dKd + kvbase * (int64_t)L * D;
    uint16_t* dVdb = a.dVd + kvbase * (int64_t)L * D;
    const int64_t dlo = (int64_t)tw_lo * L, dhi = (int64_t)(tw_hi + 1) * L;
    // Depth K and V rows of block rb as MFMA B operands.
    bf16x8 kb[1][D / 16], vb[1][D / 16];
    f32x16 gq[D / 32];   // dQ^T, depth part, of the wave's 32 query rows
    zero(gq);
    auto load = [&](int64_t rb, int buf) {
        const int64_t rl = min(rb + col, TL_rows - 1);
        const uint16_t* krow = Kdb + rl * D + 8 * hf;
        const uint16_t* vrow = Vdb + rl * D + 8 * hf;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) {
            kb[buf][si] = __builtin_bit_cast(bf16x8, ld16(krow + 16 * si));
            vb[buf][si] = __builtin_bit_cast(bf16x8, ld16(vrow + 16 * si));
        }
    };
    const int hidden = L - a.W;   // slots 0 .. hidden-1 of each token are outside the window
    auto block = [&](int64_t rb, const bf16x8 (&kr)[D / 16], const bf16x8 (&vr)[D / 16]) {
        const int64_t r = rb + col;                          // this lane's depth row
        const int rtok = (int)(min(r, TL_rows - 1) / L);
        const bool shown = (int)(r - (int64_t)rtok * L) >= hidden;
        f32x16 s, dp;
#pragma unroll
        for (int j = 0; j < 16; ++j) s[j] = dp[j] = 0.f;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) {
            s = mfma32(*(const bf16x8*)(qs + lo.a[si]), kr[si], s);
            dp = mfma32(*(const bf16x8*)(ds + lo.a[si]), vr[si], dp);
        }
        // Register j <-> query row (j/4)*8 + 4*hf + j%4; its lse2 and D from the slice.
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float4 l4 = *(const float4*)&srow[w][0][jj * 8 + 4 * hf];
            const float4 d4 = *(const float4*)&srow[w][1][jj * 8 + 4 * hf];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * jj + e;
                const int tq = (int)((fw + jj * 8 + 4 * hf + e) >> lgG);
                float p = fast_exp2(fmaf(s[j], c, -lv[e]));
                if (tq != rtok || r >= dhi || !shown) p = 0.f;
                s[j] = p;
                dp[j] = p * (dp[j] - dvv[e]);
            }
        }
        // dQ^T += Kd^T dS_d^T: Kd rows and dS_d (depth row x query) go to LDS, and both
        // operands come back through transposed reads (k = depth rows 16 sp + 8 (e/4) +
        // 4 hf + e%4 in both).
        {
            uint16_t* kslot = sout[w];
            uint16_t* tb = sds[w];
#pragma unroll
            for (int si = 0; si < D / 16; ++si)
                *(bf16x8*)(kslot + TL::off(col, 16 * si + 8 * hf)) = kr[si];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const bf16x4 v = {(__bf16)dp[4 * jj + 0], (__bf16)dp[4 * jj + 1], (__bf16)dp[4 * jj + 2],
                                  (__bf16)dp[4 * jj + 3]};
                *(bf16x4*)(tb + col * TP + 8 * jj + 4 * hf) = v;
            }
            wave_lds_sync();
            const int krow = 4 * hf + ((col & 15) >> 2), dcol = 16 * (col >> 4) + 4 * (col & 3);
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const bf16x4 b0 = lds_read_tr(tb + (krow + 16 * sp) * TP + dcol);
                const bf16x4 b1 = lds_read_tr(tb + (krow + 16 * sp + 8) * TP + dcol);
                const bf16x8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x4 a0 = lds_read_tr(kslot + TL::off(krow + 16 * sp, dcol + 32 * db));
                    const bf16x4 a1 = lds_read_tr(kslot + TL::off(krow + 16 * sp + 8, dcol + 32 * db));
                    const bf16x8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    gq[db] = mfma32(av, bv, gq[db]);
                }
            }
            wave_lds_sync();
        }
        f32x16 gv[D / 32], gk[D / 32];
        zero(gv);
        zero(gk);
        pv_block<D>(ds, 0, s, gv, lane);
        pv_block<D>(qs, 0, dp, gk, lane);
        const int nrows = (int)min((int64_t)32, dhi - rb);
        store_rows_bf16<D>(dVdb + rb * D, nrows, gv, 1.f, sout[w], lane);
        store_rows_bf16<D>(dKdb + rb * D, nrows, gk, a.scale, sout[w], lane);
    };
    for (int64_t rb = dlo; rb < dhi; rb += 32) {
        load(rb, 0);
        block(rb, kb[0], vb[0]);
    }
    // The wave's query rows' depth part of dQ (unscaled, fp32) for bwd_dq: lane column
    // col is folded row fw + col, register j of block db its element 32 db + (j/4) 8 + 4 hf + j%4.
    if (fw + col < TG) {
        const int64_t f = fw + col;
        float* drow = a.dqd + ((qhead0 + (f & (G - 1))) * T + (f >> lgG)) * D + 4 * hf;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *(float4*)(drow + 32 * db + 8 * jj) =
                    make_float4(gq[db][4 * jj + 0], gq[db][4 * jj + 1], gq[db][4 * jj + 2], gq[db][4 * jj + 3]);
    }
}

// The second stream of the current device and the two events that fork it from and join
// it to the caller's stream, created on first use and kept until the process ends.  Not
// created while the caller's stream is being captured into a graph (the pass then stays
// on that stream) or when the caller's stream belongs to another device.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool tried = false;
};
constexpr int kSideDevices = 64;
std::mutex g_side_mutex;   // guards the table and each fork ... join sequence
SideStream g_side[kSideDevices];

SideStream* side_stream(hipStream_t st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSideDevices) return nullptr;
    if (st) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(st, &sdev) != hipSuccess || sdev != dev) return nullptr;
    }
    SideStream& ss = g_side[dev];
    if (!ss.tried) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
            return nullptr;
        ss.tried = true;
        if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
            ss.stream = nullptr;
    }
    return ss.stream ? &ss : nullptr;
}

template <int D>
void launch_depth_dq(const Shape& s, BwdArgs a, hipStream_t st)
{
    const int nunits = (int)(s.B * s.Hk);
    const int64_t TG = s.T * s.G;
    if (s.L > 0) {
        constexpr int NW = 4;
        a.nblocks = (int)((TG + NW * 32 - 1) / (NW * 32));
        timing_begin("bwd_depth", st);
        hipLaunchKernelGGL((bwd_depth_kernel<D, NW>), dim3((unsigned)(nunits * a.nblocks)),
                           dim3(NW * 64), 0, st, a);
        timing_end(st);
    }
    {
        // d = 64: 4-wave workgroups, three per CU (168 registers a wave); d = 128: 8 waves.
        constexpr int NW = D == 64 ? 4 : 8;
        a.nblocks = (int)((TG + NW * 32 - 1) / (NW * 32));
        timing_begin("bwd_dq", st);
        hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)(nunits * a.nblocks)),
                           dim3(NW * 64), 0, st, a);
        timing_end(st);
    }
}

// d = 64 grids of 1024 key workgroups or more: one 8-wave workgroup of 256 keys per CU
// (two waves per SIMD), so that each staged query tile serves 8 waves rather than 4 (2-8%
// faster than two 4-wave ones).
template <int D>
bool dkdv_two_waves(const Shape& s, const DkdvPlan& pl)
{
    return D == 64 && s.B * s.Hk * pl.pieces_per_unit >= 1024;
}

template <int D>
void launch_dkdv(const Shape& s, BwdArgs a, const DkdvPlan& pl, hipStream_t st)
{
    constexpr int NW = 4;
    const int nunits = (int)(s.B * s.Hk);
    a.nkeyblocks = pl.key_blocks;
    a.piece_tiles = pl.piece_tiles;
    a.nblocks = pl.pieces_per_unit;
    const unsigned grid = (unsigned)(nunits * a.nblocks);
    timing_begin("bwd_dkdv", st);
    if (dkdv_two_waves<D>(s, pl)) {
        constexpr int NW2 = 8;
        a.nblocks = (int)((s.T + NW2 * 32 - 1) / (NW2 * 32));
        hipLaunchKernelGGL((bwd_dkdv_kernel<64, NW2, 2, false>), dim3((unsigned)(nunits * a.nblocks)),
                           dim3(NW2 * 64), 0, st, a);
    }
    else if (pl.piece_tiles > 0)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, 1, true>), dim3(grid), dim3(NW * 64), 0, st, a);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, 1, false>), dim3(grid), dim3(NW * 64), 0, st, a);
    timing_end(st);
    if (pl.piece_tiles > 0) {
        timing_begin("dkdv_reduce", st);
        hipLaunchKernelGGL((dkdv_reduce_kernel<D>), dim3((unsigned)(nunits * pl.key_blocks)),
                           dim3(256), 0, st, a);
        timing_end(st);
    }
}

template <int D>
hipError_t run(const Shape& s, BwdArgs a, hipStream_t st, bool side)
{
    {
        constexpr int RPB = 256 / (D / 8);
        timing_begin("bwd_pre", st);
        hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((a.rows + RPB - 1) / RPB)),
                           dim3(256), 0, st, a);
        timing_end(st);
    }
    const DkdvPlan pl = plan_dkdv(s);
    side = side && !dkdv_two_waves<D>(s, pl) && s.B * s.Hk * pl.key_blocks <= 1024;
    if (side) {
        std::lock_guard<std::mutex> guard(g_side_mutex);
        if (SideStream* ss = side_stream(st)) {
            hipError_t e = hipEventRecord(ss->fork, st);
            if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
            if (e != hipSuccess) return e;
            launch_depth_dq<D>(s, a, st);
            launch_dkdv<D>(s, a, pl, ss->stream);
            e = hipEventRecord(ss->join, ss->stream);
            if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->join, 0);
            if (e != hipSuccess) return e;
            return hipGetLastError();
        }
    }
    launch_depth_dq<D>(s, a, st);
    launch_dkdv<D>(s, a, pl, st);
    return hipGetLastError();
}

}  // namespace

// Small grids (under 1024 key-stationary workgroups, fewer than four per CU): every
// workgroup is resident at once and the heaviest key block -- the first, whose walk
// covers every query tile -- sets the pass's time.  Split each walk into pieces of P
// tiles, P about half a CU's share of all tiles (at least 8), when the heaviest walk is
// at least two pieces; the pieces' fp32 partials are summed by dkdv_reduce_kernel.
DkdvPlan plan_dkdv(const Shape& s)
{
    constexpr int64_t BK = 128;   // keys per workgroup of bwd_dkdv (4 waves x 32)
    DkdvPlan p;
    const int64_t TG = s.T * s.G, units = s.B * s.Hk;
    p.key_blocks = (int)((s.T + BK - 1) / BK);
    p.pieces_per_unit = p.key_blocks;
    if (units * p.key_blocks >= 1024) return p;
    auto tiles = [&](int64_t k) { return (TG - (s.noncausal ? 0 : k * BK * s.G) + BQ - 1) / BQ; };
    int64_t total = 0;
    for (int64_t k = 0; k < p.key_blocks; ++k) total += tiles(k);
    total *= units;
    const int64_t P = std::max<int64_t>(8, (total + 511) / 512);
    if (tiles(0) < 2 * P) return p;
    int64_t ppu = 0;
    for (int64_t k = 0; k < p.key_blocks; ++k) ppu += (tiles(k) + P - 1) / P;
    p.piece_tiles = (int)P;
    p.pieces_per_unit = (int)ppu;
    p.part_floats = units * ppu * 2 * BK * s.d;
    return p;
}

hipError_t launch_bwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, const void* O, const float* lse,
                           const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                           float* ws, hipStream_t st, bool side)
{
    BwdArgs a;
    a.Q = (const uint16_t*)Q;
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.Kd = (const uint16_t*)Kd;
    a.Vd = (const uint16_t*)Vd;
    a.O = (const uint16_t*)O;
    a.lse = lse;
    a.dO = (const uint16_t*)dO;
    a.dQ = (uint16_t*)dQ;
    a.dK = (uint16_t*)dK;
    a.dV = (uint16_t*)dV;
    a.dKd = (uint16_t*)dKd;
    a.dVd = (uint16_t*)dVd;
    a.rows = s.B * s.Hq * s.T;
    a.lse2 = ws;
    a.Dv = ws + a.rows;
    a.dqd = ws + ((2 * a.rows + 63) & ~int64_t(63));   // 256-byte aligned
    a.part = a.dqd + (((s.L > 0 ? a.rows * s.d : 0) + 63) & ~int64_t(63));
    a.Hq = (int)s.Hq;
    a.Hk = (int)s.Hk;
    a.T = (int)s.T;
    a.L = (int)s.L;
    a.G = s.G;
    a.W = s.W;
    a.noncausal = s.noncausal ? 1 : 0;
    a.lgG = 0;
    while ((1 << a.lgG) < s.G) ++a.lgG;
    a.c = s.scale * kLog2e;
    a.scale = s.scale;
    a.nblocks = 1;
    a.piece_tiles = 0;
    a.nkeyblocks = 0;
    return s.d == 128 ? run<128>(s, a, st, side) : run<64>(s, a, st, side);
}

}  // namespace moda
