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

__device__ __forceinline__ uint4 ld16(const void* p) { return *(const uint4*)p; }
__device__ __forceinline__ void st16(void* p, uint4 v) { *(uint4*)p = v; }

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
