// Wave-per-row MoDA kernels: the fp32 forward and backward.
//
// One wavefront handles one query row (forward), one token's G query rows
// (dQ and the token's depth gradients) or one sequence key (dK, dV).  The 64
// lanes split the head dimension; dot products are wave reductions.  These
// kernels carry no tiling: they are the straightforward GPU form of the
// operator ("Mixture-of-Depths Attention", arXiv 2603.15619, paper summary,
// section 3.4, MoDA equation with the sequence causal and depth matching
// masks) and of its derivative, used where fp32 storage is requested.  The
// variants: non-causal (every key visible) and a depth window (the last W of a
// token's L slots visible; the hidden slots get zero gradient).
#include "common.hpp"
#include "kernels.hpp"

namespace moda {
namespace {

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void stf(float* p, int64_t i, float v) { p[i] = v; }

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

struct RowArgs {
    const void* Q;
    const void* K;
    const void* V;
    const void* Kd;
    const void* Vd;
    const void* O;
    const float* lse;
    const void* dO;
    void* Oout;
    float* lse_out;
    void* dQ;
    void* dK;
    void* dV;
    void* dKd;
    void* dVd;
    float* Dws;
    int B, Hq, Hk, T, L, G;
    int W;          // visible depth slots per token (the last W of L)
    int noncausal;  // every sequence key visible
    float scale;
};

constexpr int WPB = 4;  // waves per block

// Forward: one wave per (b, h, t).
template <typename E, int D>
__global__ __launch_bounds__(WPB * 64) void fwd_rows(RowArgs a)
{
    constexpr int PE = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    const int64_t nrows = (int64_t)a.B * a.Hq * a.T;
    if (row >= nrows) return;
    const int t = (int)(row % a.T);
    const int64_t bh = row / a.T;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq), kv = h / a.G;
    const E* Q = (const E*)a.Q;
    const E* K = (const E*)a.K + ((int64_t)b * a.Hk + kv) * a.T * D;
    const E* V = (const E*)a.V + ((int64_t)b * a.Hk + kv) * a.T * D;
    float q[PE], o[PE];
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        q[i] = ldf(Q, row * D + lane + 64 * i);
        o[i] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    auto visit = [&](const E* k, const E* v) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < PE; ++i) dot += q[i] * ldf(k, lane + 64 * i);
        const float s = wave_sum(dot) * a.scale;
        const float m_new = fmaxf(m, s);
        const float alpha = __expf(m - m_new), p = __expf(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int i = 0; i < PE; ++i) o[i] = o[i] * alpha + p * ldf(v, lane + 64 * i);
        m = m_new;
    };
    const int last = a.noncausal ? a.T - 1 : t;
    for (int j = 0; j <= last; ++j) visit(K + (int64_t)j * D, V + (int64_t)j * D);
    if (a.L > 0) {
        const int64_t base = (((int64_t)b * a.Hk + kv) * a.T + t) * a.L * D;
        for (int j = a.L - a.W; j < a.L; ++j)
            visit((const E*)a.Kd + base + (int64_t)j * D, (const E*)a.Vd + base + (int64_t)j * D);
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) stf((E*)a.Oout, row * D + lane + 64 * i, o[i] / l);
    if (lane == 0) a.lse_out[row] = m + __logf(l);
}

// D = <dO, O> per row.
template <typename E, int D>
__global__ __launch_bounds__(WPB * 64) void bwd_pre(RowArgs a)
{
    constexpr int PE = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (row >= (int64_t)a.B * a.Hq * a.T) return;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < PE; ++i)
        acc += ldf((const E*)a.dO, row * D + lane + 64 * i) * ldf((const E*)a.O, row * D + lane + 64 * i);
    acc = wave_sum(acc);
    if (lane == 0) a.Dws[row] = acc;
}

// dQ of the G rows of token t and the gradients of t's L depth rows: one wave per (b, kv, t).
template <typename E, int D>
__global__ __launch_bounds__(WPB * 64) void bwd_token(RowArgs a)
{
    constexpr int PE = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t id = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (id >= (int64_t)a.B * a.Hk * a.T) return;
    const int t = (int)(id % a.T);
    const int64_t bkv = id / a.T;
    const int kv = (int)(bkv % a.Hk), b = (int)(bkv / a.Hk);
    const E* K = (const E*)a.K + bkv * a.T * D;
    const E* V = (const E*)a.V + bkv * a.T * D;
    const int64_t dbase = (bkv * a.T + t) * a.L * D;
    for (int g = 0; g < a.G; ++g) {
        const int64_t row = ((int64_t)b * a.Hq + kv * a.G + g) * a.T + t;
        float q[PE], dob[PE], dq[PE];
#pragma unroll
        for (int i = 0; i < PE; ++i) {
            q[i] = ldf((const E*)a.Q, row * D + lane + 64 * i);
            dob[i] = ldf((const E*)a.dO, row * D + lane + 64 * i);
            dq[i] = 0.f;
        }
        const float lse = a.lse[row], Dr = a.Dws[row];
        auto visit = [&](const E* k, const E* v) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                s += q[i] * ldf(k, lane + 64 * i);
                dp += dob[i] * ldf(v, lane + 64 * i);
            }
            s = wave_sum(s) * a.scale;
            dp = wave_sum(dp);
            const float ds = __expf(s - lse) * (dp - Dr);
#pragma unroll
            for (int i = 0; i < PE; ++i) dq[i] += a.scale * ds * ldf(k, lane + 64 * i);
        };
        const int last = a.noncausal ? a.T - 1 : t;
        for (int j = 0; j <= last; ++j) visit(K + (int64_t)j * D, V + (int64_t)j * D);
        for (int j = a.L - a.W; j < a.L; ++j)
            visit((const E*)a.Kd + dbase + (int64_t)j * D, (const E*)a.Vd + dbase + (int64_t)j * D);
#pragma unroll
        for (int i = 0; i < PE; ++i) stf((E*)a.dQ, row * D + lane + 64 * i, dq[i]);
    }
    for (int j = 0; j < a.L; ++j) {
        const E* kd = (const E*)a.Kd + dbase + (int64_t)j * D;
        const E* vd = (const E*)a.Vd + dbase + (int64_t)j * D;
        float dk[PE], dv[PE];
#pragma unroll
        for (int i = 0; i < PE; ++i) dk[i] = dv[i] = 0.f;
        for (int g = 0; g < a.G && j >= a.L - a.W; ++g) {   // hidden slots: zero gradient
            const int64_t row = ((int64_t)b * a.Hq + kv * a.G + g) * a.T + t;
            float s = 0.f, dp = 0.f, q[PE], dob[PE];
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                q[i] = ldf((const E*)a.Q, row * D + lane + 64 * i);
                dob[i] = ldf((const E*)a.dO, row * D + lane + 64 * i);
                s += q[i] * ldf(kd, lane + 64 * i);
                dp += dob[i] * ldf(vd, lane + 64 * i);
            }
            s = wave_sum(s) * a.scale;
            dp = wave_sum(dp);
            const float p = __expf(s - a.lse[row]);
            const float ds = p * (dp - a.Dws[row]);
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                dk[i] += a.scale * ds * q[i];
                dv[i] += p * dob[i];
            }
        }
#pragma unroll
        for (int i = 0; i < PE; ++i) {
            stf((E*)a.dKd, dbase + (int64_t)j * D + lane + 64 * i, dk[i]);
            stf((E*)a.dVd, dbase + (int64_t)j * D + lane + 64 * i, dv[i]);
        }
    }
}

// dK, dV of sequence key j: one wave per (b, kv, j).
template <typename E, int D>
__global__ __launch_bounds__(WPB * 64) void bwd_key(RowArgs a)
{
    constexpr int PE = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t id = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (id >= (int64_t)a.B * a.Hk * a.T) return;
    const int j = (int)(id % a.T);
    const int64_t bkv = id / a.T;
    const int kv = (int)(bkv % a.Hk), b = (int)(bkv / a.Hk);
    float k[PE], v[PE], dk[PE], dv[PE];
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        k[i] = ldf((const E*)a.K, id * D + lane + 64 * i);
        v[i] = ldf((const E*)a.V, id * D + lane + 64 * i);
        dk[i] = dv[i] = 0.f;
    }
    for (int g = 0; g < a.G; ++g) {
        const int64_t rb = ((int64_t)b * a.Hq + kv * a.G + g) * a.T;
        for (int t = a.noncausal ? 0 : j; t < a.T; ++t) {
            const int64_t row = rb + t;
            float s = 0.f, dp = 0.f, q[PE], dob[PE];
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                q[i] = ldf((const E*)a.Q, row * D + lane + 64 * i);
                dob[i] = ldf((const E*)a.dO, row * D + lane + 64 * i);
                s += q[i] * k[i];
                dp += dob[i] * v[i];
            }
            s = wave_sum(s) * a.scale;
            dp = wave_sum(dp);
            const float p = __expf(s - a.lse[row]);
            const float ds = p * (dp - a.Dws[row]);
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                dk[i] += a.scale * ds * q[i];
                dv[i] += p * dob[i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        stf((E*)a.dK, id * D + lane + 64 * i, dk[i]);
        stf((E*)a.dV, id * D + lane + 64 * i, dv[i]);
    }
}

inline unsigned blocks_for(int64_t waves) { return (unsigned)((waves + WPB - 1) / WPB); }

template <typename E, int D>
hipError_t run_fwd(const RowArgs& a, hipStream_t st)
{
    timing_begin("fwd_f32", st);
    hipLaunchKernelGGL((fwd_rows<E, D>), dim3(blocks_for((int64_t)a.B * a.Hq * a.T)),
                       dim3(WPB * 64), 0, st, a);
    timing_end(st);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t run_bwd(const RowArgs& a, hipStream_t st)
{
    timing_begin("bwd_pre_f32", st);
    hipLaunchKernelGGL((bwd_pre<E, D>), dim3(blocks_for((int64_t)a.B * a.Hq * a.T)),
                       dim3(WPB * 64), 0, st, a);
    timing_end(st);
    timing_begin("bwd_token_f32", st);
    hipLaunchKernelGGL((bwd_token<E, D>), dim3(blocks_for((int64_t)a.B * a.Hk * a.T)),
                       dim3(WPB * 64), 0, st, a);
    timing_end(st);
    timing_begin("bwd_key_f32", st);
    hipLaunchKernelGGL((bwd_key<E, D>), dim3(blocks_for((int64_t)a.B * a.Hk * a.T)),
                       dim3(WPB * 64), 0, st, a);
    timing_end(st);
    return hipGetLastError();
}

RowArgs make_args(const Shape& s)
{
    RowArgs a = {};
    a.B = (int)s.B;
    a.Hq = (int)s.Hq;
    a.Hk = (int)s.Hk;
    a.T = (int)s.T;
    a.L = (int)s.L;
    a.G = s.G;
    a.W = s.W;
    a.noncausal = s.noncausal ? 1 : 0;
    a.scale = s.scale;
    return a;
}

}  // namespace

hipError_t launch_fwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* Kd, const float* Vd, float* O, float* lse, hipStream_t st)
{
    RowArgs a = make_args(s);
    a.Q = Q; a.K = K; a.V = V; a.Kd = Kd; a.Vd = Vd; a.Oout = O; a.lse_out = lse;
    return s.d == 128 ? run_fwd<float, 128>(a, st) : run_fwd<float, 64>(a, st);
}

hipError_t launch_bwd_f32(const Shape& s, const float* Q, const float* K, const float* V,
                          const float* Kd, const float* Vd, const float* O, const float* lse,
                          const float* dO, float* dQ, float* dK, float* dV, float* dKd,
                          float* dVd, float* ws, hipStream_t st)
{
    RowArgs a = make_args(s);
    a.Q = Q; a.K = K; a.V = V; a.Kd = Kd; a.Vd = Vd; a.O = O; a.lse = lse; a.dO = dO;
    a.dQ = dQ; a.dK = dK; a.dV = dV; a.dKd = dKd; a.dVd = dVd; a.Dws = ws;
    return s.d == 128 ? run_bwd<float, 128>(a, st) : run_bwd<float, 64>(a, st);
}

}  // namespace moda
