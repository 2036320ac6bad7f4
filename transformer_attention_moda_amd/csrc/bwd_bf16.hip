// MoDA backward, bfloat16 storage.
#include "common.hpp"
#include "kernels.hpp"

namespace moda {

hipError_t launch_bwd_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                           const void* Kd, const void* Vd, const void* O, const float* lse,
                           const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                           float* ws, hipStream_t st)
{
    return launch_bwd_rows_bf16(s, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, ws, st);
}

}  // namespace moda
