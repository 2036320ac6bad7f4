/*
 * libmoda -- Mixture-of-Depths Attention (MoDA) on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain pointers and sizes; no C++ types or
 * exceptions cross it.
 *
 * The operator.  For batch b, query head h (KV head kv = h / G with
 * G = Hq / Hk), token t, with s = scale:
 *
 *   O[b,h,t] = softmax( s * Q[b,h,t] . [K[b,kv,0..t] || Kd[b,kv,t*L .. t*L+L-1]]^T )
 *              . [V[b,kv,0..t] || Vd[b,kv,t*L .. t*L+L-1]]
 *
 * one softmax over the causal sequence keys of the current layer and the
 * token's own L depth keys ("Mixture-of-Depths Attention", arXiv 2603.15619,
 * paper summary, section 3.4 "Mixture-of-Depths Attention (MoDA): The Unified
 * Operator": the MoDA equation, its sequence causal mask and its depth
 * matching mask).  G adjacent query heads share one KV head ("moda-attention
 * 0.1.0" PyPI page, "Key Design Choices", GQA bullet).  Depth rows are
 * token-major: row t*L + l holds token t's slot l, so a token's depth keys are
 * contiguous (paper summary, "Hardware-Efficient Implementation",
 * "Flash-compatible depth-KV layout").  With L = 0 the operator is plain causal
 * attention (same section, paragraph on the depth KV at different layers).
 *
 * Layouts (all row-major, contiguous, element type `dtype`):
 *   Q, O, dQ, dO        [B, Hq, T, d]
 *   K, V, dK, dV        [B, Hk, T, d]
 *   Kd, Vd, dKd, dVd    [B, Hk, T*L, d]
 *   lse                 [B, Hq, T]  float32 always
 * (shapes of the PyPI page's "Using the Kernel Directly").
 *
 * Ownership and execution.  All tensors are device memory owned by the
 * caller.  The library never allocates, frees or synchronises device memory;
 * each call validates its arguments on the host, enqueues its kernels on
 * `stream` (a hipStream_t; NULL means the null stream) and returns.  One
 * exception to "on `stream`": moda_bwd on a small problem runs one of its
 * kernels on a second stream of the current device, forked from `stream` by
 * an event and joined back into it by another, so work enqueued on `stream`
 * after the call is ordered after all of it, as if it had run on `stream`.
 * That stream and its two events are created by the first such call on a
 * device (not while `stream` is being captured into a graph) and kept until
 * the process ends.  Device faults surface at the caller's next
 * synchronisation.  Outputs must not alias inputs or each other.  Pointers
 * must be 16-byte aligned.
 *
 * Errors.  Every argument check runs before anything is launched; on a
 * non-OK status nothing was enqueued and outputs are untouched.
 * moda_last_error() then returns a thread-local message naming the problem.
 */
#ifndef MODA_H
#define MODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MODA_OK = 0,
    MODA_ERR_INVALID_ARGUMENT = 1, /* bad shape, pointer, alignment, scale or workspace */
    MODA_ERR_UNSUPPORTED = 2,      /* valid request outside what the library implements */
    MODA_ERR_HIP = 3               /* the HIP runtime reported an error; see moda_last_error */
} moda_status_t;

typedef enum {
    MODA_BF16 = 0, /* bfloat16 storage, fp32 accumulation, MFMA contractions */
    MODA_F32 = 1   /* fp32 storage and arithmetic throughout */
} moda_dtype_t;

/* Largest number of depth entries per token the library accepts. */
#define MODA_MAX_L 1024

/* moda_problem_t.flags bits. */
#define MODA_NONCAUSAL 1 /* every sequence key 0..T-1 is visible to every query; the depth
                            matching mask is unchanged (the MoDA README lists a non-causal
                            kernel as future work; this is the plain reading) */

typedef struct {
    int64_t B;      /* batch, >= 1 */
    int64_t Hq;     /* query heads, >= 1, multiple of Hk */
    int64_t Hk;     /* KV heads, >= 1; G = Hq / Hk must divide 32 */
    int64_t T;      /* tokens, >= 1 (any value; no multiple of a tile needed) */
    int64_t d;      /* head dimension: 64 or 128 */
    int64_t L;      /* depth entries per token, 0 .. MODA_MAX_L */
    float scale;    /* score scale, finite and > 0 (normally 1/sqrt(d)) */
    int32_t dtype;  /* moda_dtype_t */
    int32_t chunk;  /* tokens per query chunk requested; 0 = library default.
                       A tiling hint only: results do not depend on it beyond
                       fp32 summation order. */
    int32_t flags;  /* 0 or MODA_NONCAUSAL */
    int32_t window; /* depth slots visible per token: the last `window` of its L
                       slots (rows t*L + L-window .. t*L + L-1), slots being in layer
                       order so these are the most recent layers; 0 means all L.
                       0 <= window <= L.  The bounded, sliding-window depth slots of
                       the paper summary's section 6 ("Limitations and Trade-offs",
                       mitigation status). */
    int32_t reserved; /* must be 0 */
} moda_problem_t;

/*
 * Forward.  Writes O and the per-row log-sum-exp
 *   lse[b,h,t] = ln( sum over the visible keys of exp(scale * q.k) )
 * (natural log of the scaled scores; the backward pass reads it).
 * Kd and Vd may be NULL when L == 0.
 * Returns MODA_ERR_INVALID_ARGUMENT for: a NULL problem or pointer (other than
 * Kd/Vd with L == 0), a pointer not 16-byte aligned, B, Hq, Hk or T < 1,
 * Hq % Hk != 0, L < 0, a scale that is not finite or not > 0, reserved != 0,
 * chunk < 0, unknown flag bits, window < 0 or window > L, or element counts
 * that overflow int64.  Returns
 * MODA_ERR_UNSUPPORTED for d not in {64, 128}, an unknown dtype, L > MODA_MAX_L,
 * a GQA group size G that does not divide 32, T > 2^24, T*max(L, 1) >= 2^31,
 * B*Hq >= 2^31/64, or ((G-1)*T + 64)*d*2 >= 2^31 (the 32-bit byte offsets with
 * which the kernels stage a KV group's query rows).
 */
moda_status_t moda_fwd(const moda_problem_t* p, const void* Q, const void* K, const void* V,
                       const void* Kd, const void* Vd, void* O, float* lse, void* stream);

/* Bytes of device workspace moda_bwd needs for problem p (0 for an invalid p):
 * 8 bytes per query row, and for MODA_BF16 with L > 0 another 4*d bytes per
 * query row (fp32 partial gradients handed between the backward's kernels); for
 * MODA_BF16 problems too small to fill the GPU with their key blocks (fewer than
 * 1024 blocks of 128 keys over B*Hk), also 8*d bytes per key row of each piece
 * the heavy key blocks' query walks are split into (fp32 partial dK, dV). */
size_t moda_bwd_workspace_bytes(const moda_problem_t* p);

/*
 * Backward: gradients of the forward's O with respect to Q, K, V, Kd and Vd,
 * given the upstream gradient dO, the forward's O and lse (the derivative of
 * the operator above; the pages time forward+backward, MoDA README "Kernel
 * Efficiency" tables).  Every gradient is fully overwritten (dKd/dVd may be
 * NULL when L == 0).  `workspace` is caller-owned device memory of at least
 * moda_bwd_workspace_bytes(p) bytes, 256-byte aligned; it holds per-row
 * scratch between the kernels of one call, so concurrent calls need separate
 * workspaces.  Errors as for moda_fwd, plus MODA_ERR_INVALID_ARGUMENT when the
 * workspace is NULL, misaligned or smaller than required.
 */
moda_status_t moda_bwd(const moda_problem_t* p, const void* Q, const void* K, const void* V,
                       const void* Kd, const void* Vd, const void* O, const float* lse,
                       const void* dO, void* dQ, void* dK, void* dV, void* dKd, void* dVd,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moda_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The per-row scratch that moda_bwd keeps in the
 * caller's workspace lives instead in a static device array of
 * MODA_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the library's first
 * use on that GPU until the process ends.  Nothing is allocated or freed.
 * Problems whose moda_bwd_workspace_bytes exceeds that size return
 * MODA_ERR_UNSUPPORTED (at d = 128 with depth rows: about 516K query rows
 * B*Hq*T).  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams, or different host threads) race and
 * give wrong results; serialise them.  `stream` must belong to the calling
 * thread's current device.  Other arguments, results and errors as for
 * moda_bwd, which it matches bit for bit.
 */
#define MODA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

moda_status_t moda_bwd_noalloc(const moda_problem_t* p, const void* Q, const void* K,
                               const void* V, const void* Kd, const void* Vd, const void* O,
                               const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                               void* dKd, void* dVd, void* stream);

/*
 * Decoding step: one new query token per (batch, query head) at cache position
 * pos, against a cache of T tokens.  q [B, Hq, d]; K, V [B, Hk, T, d] hold the
 * sequence keys, those at positions 0..pos visible (every one of the T with
 * MODA_NONCAUSAL); Kd, Vd [B, Hk, T*L, d] hold the depth rows, of which the
 * query sees its own, rows pos*L + L-W .. pos*L + L-1 (W = window, or L).
 * Writes O [B, Hq, d] and lse [B, Hq]: exactly the forward's row at token pos
 * for the sequence that ends there (the decoding step of the paper summary's
 * "Complexity Analysis": per layer O(T d) for the sequence keys and O(L d) for
 * the depth keys).  MODA_BF16 only.  The keys are split over many workgroups
 * whose partial softmax states are merged through `workspace`: caller-owned
 * device memory of at least moda_decode_workspace_bytes(p) bytes, 256-byte
 * aligned (enough for any pos), not shared by concurrent calls.  Errors as for
 * moda_fwd, plus MODA_ERR_INVALID_ARGUMENT for pos outside 0..T-1 or a NULL,
 * misaligned or short workspace, and MODA_ERR_UNSUPPORTED for MODA_F32.
 */
size_t moda_decode_workspace_bytes(const moda_problem_t* p);

moda_status_t moda_decode(const moda_problem_t* p, int64_t pos, const void* q, const void* K,
                          const void* V, const void* Kd, const void* Vd, void* O, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Append-mode depth cache (the DepthKVCache of the PyPI page's architecture
 * list, "contiguous depth KV storage across layers"): writes one layer's entries
 * for tokens t0 .. t0+n-1, layer [B, Hk, n, d], into slot `slot` of the packed
 * token-major cache packed [B, Hk, T*L, d]: row (t0+i)*L + slot of each (b, kv)
 * block becomes layer[b, kv, i]; no other row is touched.  Appending layer l
 * into slot l for l = 0..L-1 over all tokens builds what moda_pack_depth builds
 * from the stacked layers.  A bitwise copy in p->dtype.  Requires L >= 1,
 * 0 <= slot < L, n >= 1 and t0 + n <= T; d may be any value with d * element
 * size a multiple of 16 bytes; other errors as for moda_fwd.
 */
moda_status_t moda_depth_append(const moda_problem_t* p, const void* layer, int64_t slot,
                                int64_t t0, int64_t n, void* packed, void* stream);

/*
 * Depth-KV layout packer: layer-major depth entries layers[L, B, Hk, T, d]
 * (entry l of every token contiguous, the natural per-layer layout whose
 * stride between a token's layers defeats coalescing) to the token-major
 * packed[B, Hk, T*L, d] that moda_fwd/moda_bwd read, packed row t*L + l =
 * layers[l, b, kv, t] ("Mixture-of-Depths Attention" paper summary,
 * "Hardware-Efficient Implementation": the natural layout paragraph and
 * "Flash-compatible depth-KV layout").  A bitwise copy in p->dtype.  Requires
 * L >= 1; other errors as for moda_fwd (d may be any value >= 1 with
 * d * element size a multiple of 16 bytes).
 */
moda_status_t moda_pack_depth(const moda_problem_t* p, const void* layers, void* packed,
                              void* stream);

/* Static string naming a status code. */
const char* moda_status_string(moda_status_t s);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char* moda_last_error(void);

/* Query-chunk tokens (folded query rows per workgroup / G) moda_fwd would use
 * for p, or 0 if p is invalid or unsupported. */
int32_t moda_fwd_chunk_tokens(const moda_problem_t* p);

/*
 * The forward with another choice of the depth rows each 32-row query block
 * scores (profiling support: an ablation of depth-KV layouts in the manner of
 * the paper summary's kernel ablation, Table 7 of its experiments section).
 *   MODA_SCAN_WAVE   its own tokens' rows only: what moda_fwd does (each depth
 *                    row is scored by the one wave that holds its token's G heads);
 *   MODA_SCAN_CHUNK  all rows of its workgroup's query chunk (chunk-aware layout);
 *   MODA_SCAN_ALL    all T*L rows of the KV head (flat layout, no chunking).
 * The depth matching mask keeps each query's own rows, so O and lse are those of
 * moda_fwd up to fp32 summation order; only the work and the bytes read grow.
 * MODA_BF16 only.  Errors as for moda_fwd, plus MODA_ERR_INVALID_ARGUMENT for an
 * unknown scan.
 */
#define MODA_SCAN_WAVE 0
#define MODA_SCAN_CHUNK 1
#define MODA_SCAN_ALL 2

moda_status_t moda_fwd_depth_scan(const moda_problem_t* p, int32_t scan, const void* Q,
                                  const void* K, const void* V, const void* Kd, const void* Vd,
                                  void* O, float* lse, void* stream);

/*
 * Per-kernel timing hook (profiling support; not part of the operator).
 * events: caller-created hipEvent_t handles (cast to void*), count >= 0.
 * While armed, every kernel a libmoda entry point launches on this thread is
 * bracketed by two of these events, recorded on the call's stream
 * (events[2i] before and events[2i+1] after the i-th kernel since arming), as
 * long as events remain and at most 4096 kernels per arming; further kernels
 * are not timed.  The events stay owned by the caller, who synchronises and
 * reads them (hipEventElapsedTime).
 * moda_timing_arm(NULL, 0) disarms.  Returns MODA_ERR_INVALID_ARGUMENT for a
 * negative count or NULL events with count > 0.
 */
moda_status_t moda_timing_arm(void** events, int32_t count);

/* Number of kernels bracketed since the last moda_timing_arm on this thread,
 * and the name of the i-th of them (NULL if out of range). */
int32_t moda_timing_count(void);
const char* moda_timing_label(int32_t i);

#ifdef __cplusplus
}
#endif

#endif /* MODA_H */
