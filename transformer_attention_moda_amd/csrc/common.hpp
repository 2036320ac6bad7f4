// Shared device helpers for the libmoda gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A * B + C on one 32x32x16 bf16 MFMA block.  Lane l: A row l%32 with
// k = (l/32)*8 + i; B column l%32 with the same k; D register j holds row
// (j/4)*8 + (l/32)*4 + j%4 of column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// element i of lane l is element (l%16)%4 of the 4-element chunk addressed by
// lane 4*i + (l%16)/4 of the group.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* lds_elem_ptr)
{
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_elem_ptr));
    return __builtin_bit_cast(bf16x4, r);
}

// Value reduced across the two 32-lane halves of the wave.
__device__ __forceinline__ float max_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight fp32 values to bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7)
{
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

// Row-major LDS tile of D-element bf16 rows, unpadded, with the 16-byte chunks
// of each row permuted: logical chunk c of row r sits at chunk c ^ swz(r).
//  D = 128 (a row is the 64 banks once): swz(r) = 4*(r%4) + (r/4)%4.
//  D = 64 (two rows per bank sweep):       swz(r) = 4*((r/2)%2) + (r/4)%4.
// In both, a 16-byte MFMA operand read of one chunk across 16 consecutive rows
// touches every bank once, and the 8 rows x 64 bytes of one transposed read
// (rows 8i..8i+7, chunks 4j..4j+3) cover every bank exactly twice, the minimum
// for 512 bytes.  Rows are whole 1 KiB blocks of 4 (D=128) or 8 (D=64) rows for
// the direct global->LDS loads below.
template <int D>
struct LdsTile {
    static_assert(D == 128 || D == 64, "head dimension");
    static constexpr int PITCH = D;                 // elements per row
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int RPI = 1024 / (2 * D);      // rows per 1 KiB wave load
    __device__ static __forceinline__ int swz(int row)
    {
        return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
    }
    __device__ static __forceinline__ int off(int row, int elem)
    {
        return row * D + ((((elem >> 3) ^ swz(row))) << 3) + (elem & 7);
    }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// The value of p in the first active lane, as a wave-uniform (scalar) pointer.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p)
{
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (T*)(((uint64_t)hi << 32) | lo);
}

// Direct global->LDS load of BYTES (4 or 16) per lane (buffer_load_dword[x4] ... lds):
// lane i reads base + soff + voff (byte offsets: soff wave-uniform, voff per lane, their
// sum below 2^32) and writes bytes [BYTES*i, BYTES*(i+1)) of the block at lds.  base
// and lds must be wave-uniform.  The
// buffer form is used rather than the global one because, while a global-form load
// into LDS is pending, the compiler's wait-count insertion drains every LDS read
// (lgkmcnt(0)) and every vector load (vmcnt(0)) it meets; with the buffer form it
// keeps independent reads in flight and tells apart loads into different __shared__
// arrays.  The data is in LDS once the issuing wave has waited for its vector-memory
// counter.
template <int BYTES>
__device__ __forceinline__ void buffer_load_lds(const void* base, uint32_t voff, void* lds,
                                                uint32_t soff = 0)
{
    static_assert(BYTES == 4 || BYTES == 16, "direct loads of 4 or 16 bytes per lane");
    void* b = uniform_ptr(const_cast<void*>(base));
    auto rsrc = __builtin_amdgcn_make_buffer_rsrc(b, 0, -1, 0x00020000);
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t voff, void* lds,
                                                  uint32_t soff = 0)
{
    buffer_load_lds<16>(base, voff, lds, soff);
}

// Stage rows [0, nrows) of an LdsTile<D> with direct loads.  Each wave instruction
// fills RPI rows (1 KiB); lane i fetches the logical chunk that belongs at physical
// chunk i % CPR of its row.  Tile row r is read from base + rowofs(r) elements, with
// base wave-uniform and 0 <= rowofs(r) < 2^30 - D.  Waves w, w + nw, ... share the
// instructions.
template <int D, typename RowOfs>
__device__ __forceinline__ void stage_rows(uint16_t* tile, int nrows, const uint16_t* base,
                                           RowOfs rowofs, int lane, int w, int nw)
{
    using TL = LdsTile<D>;
    const int ninstr = nrows / TL::RPI;
    const int rsub = lane / TL::CPR, p = lane % TL::CPR;
    for (int k = w; k < ninstr; k += nw) {
        const int r = k * TL::RPI + rsub;
        const int c = p ^ TL::swz(r);
        buffer_load_lds16(base, 2u * (uint32_t)(rowofs(r) + c * 8), tile + k * TL::RPI * D);
    }
}

// An opaque copy of x: the compiler cannot see that it equals x, so the values derived
// from it are computed where they are used, not kept live (or spilled) from earlier uses.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot prove threadIdx.x / 64 uniform, and every per-wave quantity derived
// from it would otherwise occupy vector registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Instruction classes for SCHED_GROUP: the compiler's scheduler places the
// next `count` instructions of the class at this point of the issue order
// (among those of the enclosing basic block), in program order of the calls.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedValu = 0x002 | 0x400;   // vector ALU including transcendentals
#define SCHED_GROUP(mask, count) __builtin_amdgcn_sched_group_barrier((mask), (count), 0)

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// acc^T += X^T P for a block of 32 rows of X held in LDS rows [row0, row0+32)
// of an LdsTile (X = V for the attention output, dO or Q for gradients).  p
// holds the 32x32 block of weights in MFMA output layout (lane column l%32,
// register j <-> row (j/4)*8 + 4*(l/32) + j%4).  X is read transposed
// (ds_read_b64_tr_b16) so that k-slot e of lane half h is row
// 16*sp + 8*(e/4) + 4*h + e%4, which is the row register 8*sp + e of p holds;
// acc[db] receives rows d = 32*db + (j/4)*8 + 4*h + j%4 of column l%32.
template <int D>
__device__ __forceinline__ void pv_block(const uint16_t* x, int row0, const f32x16& p,
                                         f32x16 (&acc)[D / 32], int lane)
{
    const int col = lane & 31, hf = lane >> 5;
    const int krow = row0 + 4 * hf + ((col & 15) >> 2);   // + 16*sp + 8*q
    const int dcol = 16 * (col >> 4) + 4 * (col & 3);      // + 32*db
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
        const bf16x8 pb = to_bf16x8(p[8 * sp + 0], p[8 * sp + 1], p[8 * sp + 2], p[8 * sp + 3],
                                    p[8 * sp + 4], p[8 * sp + 5], p[8 * sp + 6], p[8 * sp + 7]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16x4 lo = lds_read_tr(x + LdsTile<D>::off(krow + 16 * sp, dcol + 32 * db));
            const bf16x4 hi = lds_read_tr(x + LdsTile<D>::off(krow + 16 * sp + 8, dcol + 32 * db));
            const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[db] = mfma32(a, pb, acc[db]);
        }
    }
}

// Per-lane LDS element offsets inside an LdsTile<D>, computed once per kernel:
//   a[si]     the 16-byte MFMA operand chunk of row l%32, elements 16*si + 8*(l/32) .. +8
//             (A operand of K/Q/dO rows, or B operand of the same layout);
//   t[q][db]  the transposed read of pv_block: rows 8*q + 4*(l/32) + (l%16)/4,
//             elements 16*((l%32)/16) + 4*(l%4) + 32*db.
// Adding a multiple of 16 rows (16*D elements) keeps both valid, because the
// swizzle depends on the row modulo 16, so loops address tiles with per-lane
// registers plus compile-time immediates.
template <int D>
struct LaneOffsets {
    int a[D / 16];
    int t[2][D / 32];
    __device__ __forceinline__ void init(int lane)
    {
        const int col = lane & 31, hf = lane >> 5;
#pragma unroll
        for (int si = 0; si < D / 16; ++si) a[si] = LdsTile<D>::off(col, 16 * si + 8 * hf);
        const int krow = 4 * hf + ((col & 15) >> 2), dcol = 16 * (col >> 4) + 4 * (col & 3);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) t[q][db] = LdsTile<D>::off(krow + 8 * q, dcol + 32 * db);
    }
};

// pv_block with precomputed offsets: tile points at row 0 of the 32-row block
// (a multiple of 16 rows into an LdsTile<D>).
template <int D>
__device__ __forceinline__ void pv_block_pre(const uint16_t* tile, const f32x16& p,
                                             f32x16 (&acc)[D / 32], const LaneOffsets<D>& lo)
{
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
        const bf16x8 pb = to_bf16x8(p[8 * sp + 0], p[8 * sp + 1], p[8 * sp + 2], p[8 * sp + 3],
                                    p[8 * sp + 4], p[8 * sp + 5], p[8 * sp + 6], p[8 * sp + 7]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16x4 x0 = lds_read_tr(tile + lo.t[0][db] + 16 * sp * D);
            const bf16x4 x1 = lds_read_tr(tile + lo.t[1][db] + 16 * sp * D);
            const bf16x8 av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            acc[db] = mfma32(av, pb, acc[db]);
        }
    }
}

// Store a D x 32 accumulator held as acc^T blocks (lane column l%32 owns one
// output row) as bf16 row `row` of out, times `mul`: register j of block db is
// element 32*db + (j/4)*8 + 4*(l/32) + j%4.
template <int D>
__device__ __forceinline__ void store_row_bf16(uint16_t* row, const f32x16 (&acc)[D / 32],
                                               float mul, int lane)
{
    const int hf = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            bf16x4 v;
            v[0] = (__bf16)(acc[db][4 * jj + 0] * mul);
            v[1] = (__bf16)(acc[db][4 * jj + 1] * mul);
            v[2] = (__bf16)(acc[db][4 * jj + 2] * mul);
            v[3] = (__bf16)(acc[db][4 * jj + 3] * mul);
            *(bf16x4*)(row + 32 * db + 8 * jj + 4 * hf) = v;
        }
}

// The same row in fp32 (no rounding, no factor): 16-byte stores.
template <int D>
__device__ __forceinline__ void store_row_f32(float* row, const f32x16 (&acc)[D / 32], int lane)
{
    const int hf = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            *(float4*)(row + 32 * db + 8 * jj + 4 * hf) =
                make_float4(acc[db][4 * jj + 0], acc[db][4 * jj + 1], acc[db][4 * jj + 2],
                            acc[db][4 * jj + 3]);
}

template <int N>
__device__ __forceinline__ void zero(f32x16 (&a)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) a[i][j] = 0.f;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *(const uint4*)p; }
__device__ __forceinline__ void st16(void* p, uint4 v) { *(uint4*)p = v; }

// The same D x 32 accumulator (times mul, bf16) as rows [0, nrows) of the 32
// consecutive rows starting at `rows`, written through `buf` (an LdsTile<D> of 32
// rows private to the wave) so that the global stores are whole 16-byte chunks,
// RPI rows (1 KiB) per instruction, instead of 16-byte pieces of 32 rows.
template <int D>
__device__ __forceinline__ void store_rows_bf16(uint16_t* rows, int nrows, const f32x16 (&acc)[D / 32],
                                                float mul, uint16_t* buf, int lane)
{
    using TL = LdsTile<D>;
    const int col = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            bf16x4 v;
            v[0] = (__bf16)(acc[db][4 * jj + 0] * mul);
            v[1] = (__bf16)(acc[db][4 * jj + 1] * mul);
            v[2] = (__bf16)(acc[db][4 * jj + 2] * mul);
            v[3] = (__bf16)(acc[db][4 * jj + 3] * mul);
            *(bf16x4*)(buf + TL::off(col, 32 * db + 8 * jj + 4 * hf)) = v;
        }
    wave_lds_sync();
    const int rsub = lane / TL::CPR, c = lane % TL::CPR;
#pragma unroll
    for (int k = 0; k < 32 / TL::RPI; ++k) {
        const int r = k * TL::RPI + rsub;
        const uint4 v = *(const uint4*)(buf + TL::off(r, 8 * c));
        if (r < nrows) st16(rows + (int64_t)r * D + 8 * c, v);
    }
    wave_lds_sync();
}

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
template <int D, int NB, bool SUM = true>
__device__ __forceinline__ void softmax_update(f32x16 (&s)[2], float& m, float& l,
                                               f32x16 (&o)[D / 32], float c)
{
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
    mt = max_halves(mt);
    const bool grow = (mt - m) * c > kRescaleLog2;   // true for the first visible score
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
    if (SUM) l += sum_halves(ps);
}

// Workgroup id -> logical work index.  Workgroups are dispatched to the 8 XCDs
// round-robin (id % 8); this gives XCD x the contiguous logical range
// [start(x), start(x) + count(x)), so that an XCD's L2 sees the same KV head
// for many consecutive workgroups.
__device__ __forceinline__ int xcd_remap(int id, int n)
{
    const int x = id & 7, k = id >> 3, q = n >> 3, r = n & 7;
    const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return start + k;
}

}  // namespace moda
