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
    bool noncausal;  // every sequence key visible to every query
    int W;           // visible depth slots per token: the last W of L (W == L: all)
};

// Forward, bfloat16 storage, MFMA.  rows_per_wg is 128 or 256 folded query rows;
// scan selects the depth rows a wave scores (0: its own tokens'; 1, 2: the ablation's
// chunk-wide and all-rows scans).
hipError_t launch_fwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, void* O, float* lse, int rows_per_wg,
                           hipStream_t st, int scan = 0);

// The key-stationary backward pass on small grids: a key block's walk over the query
// tiles split into pieces of piece_tiles tiles (0: not split), pieces_per_unit work blocks
// per (b, kv); part_floats fp32 of partial dK, dV in the workspace.
struct DkdvPlan {
    int piece_tiles = 0;
    int key_blocks = 0;
    int pieces_per_unit = 0;
    int64_t part_floats = 0;
};
DkdvPlan plan_dkdv(const Shape& s);

// Backward, bfloat16 storage.  ws: the workspace (lse2 and D per row, the depth part of
// dQ when L > 0, then the split pass's partials; sizes as the ABI's workspace query).
// side: small problems may run the key-stationary pass on the device's second stream,
// forked from and joined back into st (false keeps every launch on st).
hipError_t launch_bwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, const void* O, const float* lse,
                           const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                           float* ws, hipStream_t st, bool side);

// fp32 forward / backward (plain wave-per-row kernels).
hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* Kd, const float* Vd, float* O, float* lse, hipStream_t st);
hipError_t launch_bwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* Kd, const float* Vd, const float* O, const float* lse,
                          const float* dO, float* dQ, float* dK, float* dV, float* dKd,
                          float* dVd, float* ws, hipStream_t st);

// Decoding step (bfloat16): how the visible keys of one query token are split into
// partials, and the launch.  nseq: visible sequence keys.
struct DecodePlan {
    int64_t nblk_seq, nblk;   // 32-row blocks: sequence, then depth
    int64_t nsplit;           // workgroups per (b, kv)
    int64_t o_floats, ml_floats;
};
DecodePlan plan_decode(const Shape& s, int64_t nseq);
size_t decode_ws_bytes(const DecodePlan& pl);
hipError_t launch_decode_bf16(const Shape& s, int64_t pos, const void* q, const void* K,
                              const void* V, const void* Kd, const void* Vd, void* O, float* lse,
                              void* ws, hipStream_t st);

// Depth-cache append: layer [B, Hk, n, row_bytes] -> rows (t0+i)*L + slot of
// packed [B, Hk, T*L, row_bytes].
hipError_t launch_depth_append(int64_t B, int64_t Hk, int64_t T, int64_t L, int64_t row_bytes,
                               int64_t slot, int64_t t0, int64_t n, const void* layer,
                               void* packed, hipStream_t st);

// Depth packer: [L, B, Hk, T, row_bytes] -> [B, Hk, T*L, row_bytes].
hipError_t launch_pack_depth(int64_t L, int64_t B, int64_t Hk, int64_t T, int64_t row_bytes,
                             const void* layers, void* packed, hipStream_t st);

}  // namespace moda
