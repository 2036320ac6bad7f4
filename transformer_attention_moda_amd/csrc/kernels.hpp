// Host-side launchers of the libmoda kernels (internal; the C ABI in
// include/moda.h validates arguments before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {

// Timing hook: bracket one kernel launch with the caller's events, if armed.
void timing_begin(const char* label, hipStream_t st);
void timing_end(hipStream_t st);

struct Shape {
    int64_t B, Hq, Hk, T, d, L;
    float scale;
    int G;
};

// Forward, bfloat16 storage, MFMA.  rows_per_wg is 128 or 256 folded query rows.
hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, void* O, float* lse, int rows_per_wg,
                           hipStream_t st);

// Backward, bfloat16 storage.  ws: B*Hq*T floats.
hipError_t launch_bwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, const void* O, const float* lse,
                           const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                           float* ws, hipStream_t st);

// fp32 forward / backward (plain wave-per-row kernels).
hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* Kd, const float* Vd, float* O, float* lse, hipStream_t st);
hipError_t launch_bwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* Kd, const float* Vd, const float* O, const float* lse,
                          const float* dO, float* dQ, float* dK, float* dV, float* dKd,
                          float* dVd, float* ws, hipStream_t st);

// Depth packer: [L, B, Hk, T, row_bytes] -> [B, Hk, T*L, row_bytes].
hipError_t launch_pack_depth(int64_t L, int64_t B, int64_t Hk, int64_t T, int64_t row_bytes,
                             const void* layers, void* packed, hipStream_t st);

}  // namespace moda
