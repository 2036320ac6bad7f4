// libmoda C ABI: argument validation and dispatch (see include/moda.h).
//
// Every check below runs on the host before anything is enqueued, so an
// invalid call returns its status without touching the device.
#include "moda.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

moda_status_t fail(moda_status_t s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest sizes the kernels' 32-bit token and row indices accept.
constexpr int64_t kMaxT = int64_t(1) << 24;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

int64_t elem_size(int32_t dtype) { return dtype == MODA_BF16 ? 2 : 4; }

bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Common shape checks.  need_head_dim: d must be 64 or 128 (attention kernels).
moda_status_t check_problem(const moda_problem_t* p, bool need_head_dim, moda::Shape* s)
{
    if (!p) return fail(MODA_ERR_INVALID_ARGUMENT, "problem pointer is NULL");
    if (p->B < 1 || p->Hq < 1 || p->Hk < 1 || p->T < 1 || p->d < 1)
        return fail(MODA_ERR_INVALID_ARGUMENT, "B, Hq, Hk, T and d must be >= 1 (got %lld %lld %lld %lld %lld)",
                    (long long)p->B, (long long)p->Hq, (long long)p->Hk, (long long)p->T,
                    (long long)p->d);
    if (p->Hq % p->Hk != 0)
        return fail(MODA_ERR_INVALID_ARGUMENT, "Hq (%lld) is not a multiple of Hk (%lld)",
                    (long long)p->Hq, (long long)p->Hk);
    if (p->L < 0) return fail(MODA_ERR_INVALID_ARGUMENT, "L must be >= 0 (got %lld)", (long long)p->L);
    if (!std::isfinite(p->scale) || !(p->scale > 0.f))
        return fail(MODA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (p->reserved != 0) return fail(MODA_ERR_INVALID_ARGUMENT, "reserved field must be 0");
    if (p->chunk < 0) return fail(MODA_ERR_INVALID_ARGUMENT, "chunk must be >= 0");
    if (p->flags & ~MODA_NONCAUSAL)
        return fail(MODA_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", (unsigned)p->flags);
    if (p->window < 0 || p->window > p->L)
        return fail(MODA_ERR_INVALID_ARGUMENT, "window %d outside 0..L (L = %lld)", (int)p->window,
                    (long long)p->L);
    if (p->dtype != MODA_BF16 && p->dtype != MODA_F32)
        return fail(MODA_ERR_UNSUPPORTED, "unknown dtype %d", (int)p->dtype);
    int64_t n = 0;
    if (!mul_ok(p->B, p->Hq, &n) || !mul_ok(n, p->T, &n) || !mul_ok(n, p->d, &n) ||
        !mul_ok(n, elem_size(p->dtype), &n) || !mul_ok(p->B, p->Hk, &n) || !mul_ok(n, p->T, &n) ||
        !mul_ok(n, p->L > 0 ? p->L : 1, &n) || !mul_ok(n, p->d, &n) ||
        !mul_ok(n, elem_size(p->dtype), &n))
        return fail(MODA_ERR_INVALID_ARGUMENT, "tensor sizes overflow int64");
    if (need_head_dim && p->d != 64 && p->d != 128)
        return fail(MODA_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                    (long long)p->d);
    if (p->L > MODA_MAX_L)
        return fail(MODA_ERR_UNSUPPORTED, "L = %lld exceeds MODA_MAX_L = %d", (long long)p->L,
                    MODA_MAX_L);
    const int64_t G = p->Hq / p->Hk;
    if (32 % G != 0)
        return fail(MODA_ERR_UNSUPPORTED, "GQA group size G = %lld must divide 32", (long long)G);
    if (p->T > kMaxT || p->T * (p->L > 0 ? p->L : 1) > kMaxRows || p->B * p->Hq > kMaxRows / 64)
        return fail(MODA_ERR_UNSUPPORTED, "sizes beyond the kernels' 32-bit row indices");
    // The backward stages a KV group's query rows (G heads of T rows) with 32-bit byte
    // offsets from the tile's first row; they reach (G-1)*T + 64 rows.
    if (((G - 1) * p->T + 64) * p->d * 2 >= (int64_t(1) << 31))
        return fail(MODA_ERR_UNSUPPORTED,
                    "(G-1)*T = %lld rows of d = %lld exceed the 2 GiB reach of the staging offsets",
                    (long long)((G - 1) * p->T), (long long)p->d);
    if (s) {
        s->B = p->B; s->Hq = p->Hq; s->Hk = p->Hk; s->T = p->T; s->d = p->d; s->L = p->L;
        s->scale = p->scale;
        s->G = (int)G;
        s->noncausal = (p->flags & MODA_NONCAUSAL) != 0;
        s->W = p->window > 0 ? p->window : (int)p->L;
    }
    return MODA_OK;
}

moda_status_t check_ptr(const void* ptr, const char* name)
{
    if (!ptr) return fail(MODA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (!aligned16(ptr)) return fail(MODA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
    return MODA_OK;
}

moda_status_t check_depth(const moda_problem_t* p, const void* a, const char* na, const void* b,
                          const char* nb)
{
    if (p->L == 0) {
        if ((a && !aligned16(a)) || (b && !aligned16(b)))
            return fail(MODA_ERR_INVALID_ARGUMENT, "%s/%s not 16-byte aligned", na, nb);
        return MODA_OK;
    }
    moda_status_t st = check_ptr(a, na);
    if (st != MODA_OK) return st;
    return check_ptr(b, nb);
}

moda_status_t hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return MODA_OK;
    return fail(MODA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int rows_per_workgroup(const moda_problem_t* p, int G)
{
    // Default: 256 folded rows (8 waves, two per SIMD) at d = 128; 128 rows at d = 64, whose
    // 4-wave workgroups fit three per CU (168 registers a wave, three waves per SIMD).
    if (p->chunk == 0) return p->d == 64 ? 128 : 256;
    return (int64_t)p->chunk * G >= 256 ? 256 : 128;
}

// Two fp32 values per query row: the log-sum-exp in log2 units and D = <dO, O>;
// in bfloat16 with depth rows, then (256-byte aligned) an fp32 row of d values per
// query row: the depth rows' part of dQ, passed from bwd_depth to bwd_dq; then, for
// bfloat16 problems whose key pass is split (small grids), the pieces' partial dK, dV.
size_t bwd_ws_bytes(const moda::Shape& s, int32_t dtype)
{
    const size_t rows = (size_t)(s.B * s.Hq * s.T);
    size_t n = (2 * rows * sizeof(float) + 255) & ~size_t(255);
    if (dtype == MODA_BF16 && s.L > 0) n += rows * (size_t)s.d * sizeof(float);
    n = (n + 255) & ~size_t(255);
    // bfloat16 on small grids: the split key-stationary pass's fp32 partial dK, dV.
    if (dtype == MODA_BF16) n += (size_t)moda::plan_dkdv(s).part_floats * sizeof(float);
    return (n + 255) & ~size_t(255);
}

// ---- scratch of the no-allocation backward ----
// One static device array per GPU (the code object's copy on that device), used by
// moda_bwd_noalloc in place of the caller's workspace.  In host code the name
// `scratch` is a host-side stand-in, not a device address; the address on each
// device comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[MODA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device, which `st` must belong to.
moda_status_t device_scratch(hipStream_t st, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MODA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (st) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(st, &sdev);
        if (e != hipSuccess) return fail(MODA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(MODA_ERR_INVALID_ARGUMENT,
                        "stream belongs to device %d, not to the current device %d", (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MODA_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = ptr;
    });
    if (g_scratch_err[dev] != hipSuccess)
        return fail(MODA_ERR_HIP, "hipGetSymbolAddress(scratch): %s",
                    hipGetErrorString(g_scratch_err[dev]));
    if (!g_scratch_ptr[dev]) return fail(MODA_ERR_HIP, "no device address for the scratch array");
    *out = g_scratch_ptr[dev];
    return MODA_OK;
}

constexpr int32_t kMaxTimedKernels = 4096;

struct Timing {
    hipEvent_t* events = nullptr;
    int32_t count = 0;
    int32_t used = 0;   // events recorded
    const char* labels[kMaxTimedKernels];
    int32_t nlabels = 0;
};
thread_local Timing g_timing;

// Problem and pointer checks shared by the two backward entry points.
moda_status_t check_bwd(const moda_problem_t* p, const void* Q, const void* K, const void* V,
                        const void* Kd, const void* Vd, const void* O, const float* lse,
                        const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                        moda::Shape* s)
{
    moda_status_t st = check_problem(p, true, s);
    if (st != MODA_OK) return st;
    const void* ptrs[] = {Q, K, V, O, lse, dO, dQ, dK, dV};
    const char* names[] = {"Q", "K", "V", "O", "lse", "dO", "dQ", "dK", "dV"};
    for (int i = 0; i < 9; ++i)
        if ((st = check_ptr(ptrs[i], names[i])) != MODA_OK) return st;
    if ((st = check_depth(p, Kd, "Kd", Vd, "Vd")) != MODA_OK) return st;
    return check_depth(p, dKd, "dKd", dVd, "dVd");
}

moda_status_t launch_bwd(const moda_problem_t* p, const moda::Shape& s, const void* Q,
                         const void* K, const void* V, const void* Kd, const void* Vd,
                         const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                         void* dV, void* dKd, void* dVd, void* ws, hipStream_t hs, bool side)
{
    hipError_t e;
    if (p->dtype == MODA_BF16)
        e = moda::launch_bwd_bf16(s, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd,
                                  (float*)ws, hs, side);
    else
        e = moda::launch_bwd_f32(s, (const float*)Q, (const float*)K, (const float*)V,
                                 (const float*)Kd, (const float*)Vd, (const float*)O, lse,
                                 (const float*)dO, (float*)dQ, (float*)dK, (float*)dV,
                                 (float*)dKd, (float*)dVd, (float*)ws, hs);
    return hip_status(e, "moda_bwd launch");
}

}  // namespace

namespace moda {

void timing_begin(const char* label, hipStream_t st)
{
    Timing& t = g_timing;
    // A kernel is timed only while both of its events and a label slot remain, so that
    // every bracketed kernel has a label.
    if (!t.events || t.used + 2 > t.count || t.nlabels >= kMaxTimedKernels) return;
    (void)hipEventRecord(t.events[t.used++], st);
    t.labels[t.nlabels++] = label;
}

void timing_end(hipStream_t st)
{
    Timing& t = g_timing;
    if (!t.events || t.used % 2 == 0) return;
    (void)hipEventRecord(t.events[t.used++], st);
}

}  // namespace moda

extern "C" {

moda_status_t moda_timing_arm(void** events, int32_t count)
{
    if (count < 0 || (count > 0 && !events))
        return fail(MODA_ERR_INVALID_ARGUMENT, "bad timing event array");
    g_timing.events = count > 0 ? reinterpret_cast<hipEvent_t*>(events) : nullptr;
    g_timing.count = count;
    g_timing.used = 0;
    g_timing.nlabels = 0;
    return MODA_OK;
}

int32_t moda_timing_count(void) { return g_timing.used / 2; }

const char* moda_timing_label(int32_t i)
{
    if (i < 0 || i >= g_timing.used / 2) return nullptr;
    return g_timing.labels[i];
}


const char* moda_status_string(moda_status_t s)
{
    switch (s) {
    case MODA_OK: return "MODA_OK";
    case MODA_ERR_INVALID_ARGUMENT: return "MODA_ERR_INVALID_ARGUMENT";
    case MODA_ERR_UNSUPPORTED: return "MODA_ERR_UNSUPPORTED";
    case MODA_ERR_HIP: return "MODA_ERR_HIP";
    }
    return "unknown moda_status_t";
}

const char* moda_last_error(void) { return g_err; }

int32_t moda_fwd_chunk_tokens(const moda_problem_t* p)
{
    moda::Shape s;
    if (check_problem(p, true, &s) != MODA_OK) return 0;
    if (p->dtype == MODA_F32) return 1;
    return rows_per_workgroup(p, s.G) / s.G;
}

moda_status_t moda_fwd(const moda_problem_t* p, const void* Q, const void* K, const void* V,
                       const void* Kd, const void* Vd, void* O, float* lse, void* stream)
{
    moda::Shape s;
    moda_status_t st = check_problem(p, true, &s);
    if (st != MODA_OK) return st;
    const void* ptrs[] = {Q, K, V, O, lse};
    const char* names[] = {"Q", "K", "V", "O", "lse"};
    for (int i = 0; i < 5; ++i)
        if ((st = check_ptr(ptrs[i], names[i])) != MODA_OK) return st;
    if ((st = check_depth(p, Kd, "Kd", Vd, "Vd")) != MODA_OK) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (p->dtype == MODA_BF16)
        e = moda::launch_fwd_bf16(s, Q, K, V, Kd, Vd, O, lse, rows_per_workgroup(p, s.G), hs);
    else
        e = moda::launch_fwd_f32(s, (const float*)Q, (const float*)K, (const float*)V,
                                 (const float*)Kd, (const float*)Vd, (float*)O, lse, hs);
    return hip_status(e, "moda_fwd launch");
}

moda_status_t moda_fwd_depth_scan(const moda_problem_t* p, int32_t scan, const void* Q,
                                  const void* K, const void* V, const void* Kd, const void* Vd,
                                  void* O, float* lse, void* stream)
{
    if (scan < MODA_SCAN_WAVE || scan > MODA_SCAN_ALL)
        return fail(MODA_ERR_INVALID_ARGUMENT, "unknown depth scan %d", (int)scan);
    moda::Shape s;
    moda_status_t st = check_problem(p, true, &s);
    if (st != MODA_OK) return st;
    if (p->dtype != MODA_BF16)
        return fail(MODA_ERR_UNSUPPORTED, "the depth-scan ablation is built for MODA_BF16 only");
    const void* ptrs[] = {Q, K, V, O, lse};
    const char* names[] = {"Q", "K", "V", "O", "lse"};
    for (int i = 0; i < 5; ++i)
        if ((st = check_ptr(ptrs[i], names[i])) != MODA_OK) return st;
    if ((st = check_depth(p, Kd, "Kd", Vd, "Vd")) != MODA_OK) return st;
    return hip_status(moda::launch_fwd_bf16(s, Q, K, V, Kd, Vd, O, lse, rows_per_workgroup(p, s.G),
                                            reinterpret_cast<hipStream_t>(stream), scan),
                      "moda_fwd_depth_scan launch");
}

size_t moda_bwd_workspace_bytes(const moda_problem_t* p)
{
    moda::Shape s;
    if (check_problem(p, true, &s) != MODA_OK) return 0;
    return bwd_ws_bytes(s, p->dtype);
}

moda_status_t moda_bwd(const moda_problem_t* p, const void* Q, const void* K, const void* V,
                       const void* Kd, const void* Vd, const void* O, const float* lse,
                       const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    moda::Shape s;
    moda_status_t st = check_bwd(p, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, &s);
    if (st != MODA_OK) return st;
    if (!workspace) return fail(MODA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(MODA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    const size_t need = bwd_ws_bytes(s, p->dtype);
    if (workspace_bytes < need)
        return fail(MODA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    return launch_bwd(p, s, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, workspace,
                      reinterpret_cast<hipStream_t>(stream), true);
}

moda_status_t moda_bwd_noalloc(const moda_problem_t* p, const void* Q, const void* K,
                               const void* V, const void* Kd, const void* Vd, const void* O,
                               const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                               void* dKd, void* dVd, void* stream)
{
    moda::Shape s;
    moda_status_t st = check_bwd(p, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, &s);
    if (st != MODA_OK) return st;
    const size_t need = bwd_ws_bytes(s, p->dtype);
    if (need > MODA_NOALLOC_SCRATCH_BYTES)
        return fail(MODA_ERR_UNSUPPORTED,
                    "problem needs %zu bytes of scratch; moda_bwd_noalloc has %zu (use moda_bwd)",
                    need, (size_t)MODA_NOALLOC_SCRATCH_BYTES);
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if ((st = device_scratch(hs, &ws)) != MODA_OK) return st;
    // The kernels write every scratch value they read (per-row lse and D first, then
    // the depth part of dQ), so nothing needs clearing between calls.
    // Every launch stays on the caller's stream: no stream or event is created here.
    return launch_bwd(p, s, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, ws, hs, false);
}

size_t moda_decode_workspace_bytes(const moda_problem_t* p)
{
    moda::Shape s;
    if (check_problem(p, true, &s) != MODA_OK || p->dtype != MODA_BF16) return 0;
    // The split grows with the number of visible keys: the whole cache bounds it.
    return moda::decode_ws_bytes(moda::plan_decode(s, s.T));
}

moda_status_t moda_decode(const moda_problem_t* p, int64_t pos, const void* q, const void* K,
                          const void* V, const void* Kd, const void* Vd, void* O, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    moda::Shape s;
    moda_status_t st = check_problem(p, true, &s);
    if (st != MODA_OK) return st;
    if (p->dtype != MODA_BF16)
        return fail(MODA_ERR_UNSUPPORTED, "moda_decode is built for MODA_BF16 only");
    if (pos < 0 || pos >= p->T)
        return fail(MODA_ERR_INVALID_ARGUMENT, "pos = %lld outside the cache of T = %lld tokens",
                    (long long)pos, (long long)p->T);
    const void* ptrs[] = {q, K, V, O, lse};
    const char* names[] = {"q", "K", "V", "O", "lse"};
    for (int i = 0; i < 5; ++i)
        if ((st = check_ptr(ptrs[i], names[i])) != MODA_OK) return st;
    if ((st = check_depth(p, Kd, "Kd", Vd, "Vd")) != MODA_OK) return st;
    if (!workspace) return fail(MODA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(MODA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    const size_t need = moda::decode_ws_bytes(moda::plan_decode(s, s.noncausal ? s.T : pos + 1));
    if (workspace_bytes < need)
        return fail(MODA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu required",
                    workspace_bytes, need);
    return hip_status(moda::launch_decode_bf16(s, pos, q, K, V, Kd, Vd, O, lse, workspace,
                                               reinterpret_cast<hipStream_t>(stream)),
                      "moda_decode launch");
}

moda_status_t moda_depth_append(const moda_problem_t* p, const void* layer, int64_t slot,
                                int64_t t0, int64_t n, void* packed, void* stream)
{
    moda::Shape s;
    moda_status_t st = check_problem(p, false, &s);
    if (st != MODA_OK) return st;
    if (p->L < 1) return fail(MODA_ERR_INVALID_ARGUMENT, "moda_depth_append needs L >= 1");
    if (slot < 0 || slot >= p->L)
        return fail(MODA_ERR_INVALID_ARGUMENT, "slot %lld outside 0..L-1 (L = %lld)",
                    (long long)slot, (long long)p->L);
    if (n < 1 || t0 < 0 || t0 > p->T - n)
        return fail(MODA_ERR_INVALID_ARGUMENT, "tokens %lld..%lld outside the cache of T = %lld",
                    (long long)t0, (long long)(t0 + n - 1), (long long)p->T);
    const int64_t row_bytes = p->d * elem_size(p->dtype);
    if (row_bytes % 16 != 0)
        return fail(MODA_ERR_UNSUPPORTED, "row of %lld bytes is not a multiple of 16",
                    (long long)row_bytes);
    if ((st = check_ptr(layer, "layer")) != MODA_OK) return st;
    if ((st = check_ptr(packed, "packed")) != MODA_OK) return st;
    return hip_status(moda::launch_depth_append(p->B, p->Hk, p->T, p->L, row_bytes, slot, t0, n,
                                                layer, packed,
                                                reinterpret_cast<hipStream_t>(stream)),
                      "moda_depth_append launch");
}

moda_status_t moda_pack_depth(const moda_problem_t* p, const void* layers, void* packed,
                              void* stream)
{
    moda::Shape s;
    moda_status_t st = check_problem(p, false, &s);
    if (st != MODA_OK) return st;
    if (p->L < 1) return fail(MODA_ERR_INVALID_ARGUMENT, "moda_pack_depth needs L >= 1");
    const int64_t row_bytes = p->d * elem_size(p->dtype);
    if (row_bytes % 16 != 0)
        return fail(MODA_ERR_UNSUPPORTED, "row of %lld bytes is not a multiple of 16",
                    (long long)row_bytes);
    if ((st = check_ptr(layers, "layers")) != MODA_OK) return st;
    if ((st = check_ptr(packed, "packed")) != MODA_OK) return st;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    return hip_status(moda::launch_pack_depth(p->L, p->B, p->Hk, p->T, row_bytes, layers, packed, hs),
                      "moda_pack_depth launch");
}

}  // extern "C"
