/*
 * CPU oracle for the Mixture-of-Depths Attention (MoDA) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table with
 * the HIP library; the two meet only through seeded inputs.
 *
 * What it computes is the plain definition of the operator, written out with
 * fp64 arithmetic and a two-pass softmax per query row:
 *
 *   MoDA(Q_h, K, V, K_depth, V_depth) = softmax(Q_h [K || K_depth]^T / sqrt(d) + M) [V || V_depth]
 *
 * from "Mixture-of-Depths Attention" (arXiv 2603.15619, paper summary),
 * section 3.4 "Mixture-of-Depths Attention (MoDA): The Unified Operator", the
 * MoDA equation, with the two masks of the same section:
 *   - sequence causal mask: key j is visible to the query at token t iff j <= t
 *     (first masking bullet; under GQA the folded form floor(i_q/G) >= i_k);
 *   - depth matching mask: flattened depth row r is visible iff floor(r/L) = t
 *     (second masking bullet, floor(i_q/G) = floor(j_d/L)), i.e. a token sees
 *     exactly its own L depth rows t*L .. t*L+L-1 (same summary, "Flash-compatible
 *     depth-KV layout").
 * GQA head mapping: G = Hq/Hk adjacent query heads share one KV head, so query
 * head h reads KV head h / G ("moda-attention 0.1.0" PyPI page, "Key Design
 * Choices", GQA bullet, which expands KV with repeat_interleave; paper summary,
 * "Group-aware depth-KV calculation").
 * Tensor shapes follow the PyPI page, "Using the Kernel Directly":
 *   Q [B,Hq,T,d], K/V [B,Hk,T,d], K_depth/V_depth [B,Hk,T*L,d].
 *
 * The score scale is passed in (the kernel ABI passes 1/sqrt(d) as an fp32
 * value; the tests pass that same value).  The log-sum-exp returned per row is
 * m + ln(Z) over the scaled scores (natural log) -- a convention of this
 * library's interface, not something the pages define.
 *
 * The backward pass is the derivative of the definition above (the pages time
 * forward+backward but print no backward formulas):
 *   p_j = exp(s_j - lse), q_l = exp(u_l - lse), D = <dO, O>
 *   ds_j = p_j (<dO, V_j> - D),  du_l = q_l (<dO, Vd_{t,l}> - D)
 *   dQ   = scale (sum_j ds_j K_j + sum_l du_l Kd_{t,l})
 *   dK_j += scale ds_j Q,  dV_j += p_j dO,  dKd_{t,l} += scale du_l Q,  dVd_{t,l} += q_l dO
 *
 * Two variants of the masks, both readings of open items on the pages:
 *   - non-causal (flag bit 0): every sequence key 0 .. T-1 is visible to every
 *     query; the depth matching mask is unchanged.  The MoDA README lists a
 *     non-causal kernel as future work without defining it; dropping the
 *     sequence causal mask and keeping the depth one is the plain reading.
 *   - depth window W (0 < W <= L; 0 means L): a token sees only the last W of
 *     its L depth slots, rows t*L + L-W .. t*L + L-1.  The paper summary's
 *     section 6 ("Limitations and Trade-offs", mitigation status) sketches
 *     bounded depth-KV slots with a sliding-window recency policy; slots are in
 *     layer order, so the last W are the most recent layers.
 *
 * Element storage codes: 0 = bf16 (raw 16-bit patterns, upcast exactly),
 * 1 = fp32, 2 = fp64.  All arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, Hq, Hk, T, d, L;
    double scale;
    int32_t dtype;    /* storage code of Q, K, V, K_depth, V_depth, dO */
    int32_t flags;    /* bit 0: non-causal */
    int64_t window;   /* visible depth slots per token (the last ones); 0 = all L */
} oracle_shape;

/* Last sequence key visible to the query at token t. */
static int64_t last_key(const oracle_shape* s, int64_t t)
{
    return (s->flags & 1) ? s->T - 1 : t;
}

/* First visible depth slot of a token (slots first_slot .. L-1 are visible). */
static int64_t first_slot(const oracle_shape* s)
{
    return s->window > 0 ? s->L - s->window : 0;
}

static double elem(const void* p, int dtype, int64_t i)
{
    if (dtype == 2) return ((const double*)p)[i];
    if (dtype == 1) return (double)((const float*)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Flat element offsets of row starts. */
static int64_t q_off(const oracle_shape* s, int64_t b, int64_t h, int64_t t)
{
    return ((b * s->Hq + h) * s->T + t) * s->d;
}
static int64_t kv_off(const oracle_shape* s, int64_t b, int64_t kv, int64_t j)
{
    return ((b * s->Hk + kv) * s->T + j) * s->d;
}
static int64_t dep_off(const oracle_shape* s, int64_t b, int64_t kv, int64_t r)
{
    return ((b * s->Hk + kv) * s->T * s->L + r) * s->d;
}

static double dot(const oracle_shape* s, const void* x, int64_t xo, const void* y, int64_t yo)
{
    double acc = 0.0;
    for (int64_t e = 0; e < s->d; ++e)
        acc += elem(x, s->dtype, xo + e) * elem(y, s->dtype, yo + e);
    return acc;
}

/*
 * One query row (b, h, t): its visible sequence scores (keys 0 .. last_key)
 * and its visible depth scores (slots first_slot .. L-1 of token t), one
 * softmax over their concatenation, the output row and the log-sum-exp.
 * `scores` is caller scratch of length T+L.
 */
static void row_forward(const oracle_shape* s, const void* Q, const void* K, const void* V,
                        const void* Kd, const void* Vd, int64_t b, int64_t h, int64_t t,
                        double* scores, double* o, double* lse)
{
    const int64_t G = s->Hq / s->Hk, kv = h / G, L = s->L, d = s->d;
    const int64_t qo = q_off(s, b, h, t);
    const int64_t nseq = last_key(s, t) + 1, l0 = first_slot(s);
    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < nseq; ++j) {
        scores[j] = s->scale * dot(s, Q, qo, K, kv_off(s, b, kv, j));
        if (scores[j] > m) m = scores[j];
    }
    for (int64_t l = l0; l < L; ++l) {
        scores[nseq + l] = s->scale * dot(s, Q, qo, Kd, dep_off(s, b, kv, t * L + l));
        if (scores[nseq + l] > m) m = scores[nseq + l];
    }
    /* pass 2: weights, denominator, weighted sum of values */
    double Z = 0.0;
    for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t j = 0; j < nseq; ++j) {
        const double w = exp(scores[j] - m);
        const int64_t vo = kv_off(s, b, kv, j);
        Z += w;
        for (int64_t e = 0; e < d; ++e) o[e] += w * elem(V, s->dtype, vo + e);
    }
    for (int64_t l = l0; l < L; ++l) {
        const double w = exp(scores[nseq + l] - m);
        const int64_t vo = dep_off(s, b, kv, t * L + l);
        Z += w;
        for (int64_t e = 0; e < d; ++e) o[e] += w * elem(Vd, s->dtype, vo + e);
    }
    for (int64_t e = 0; e < d; ++e) o[e] /= Z;
    *lse = m + log(Z);
}

static int shape_ok(const oracle_shape* s)
{
    return s && s->B > 0 && s->Hq > 0 && s->Hk > 0 && s->T > 0 && s->d > 0 && s->L >= 0 &&
           s->Hq % s->Hk == 0 && s->dtype >= 0 && s->dtype <= 2 && (s->flags & ~1) == 0 &&
           s->window >= 0 && s->window <= s->L;
}

/*
 * Forward for a list of query rows.  rows holds nrows triples (b, h, t);
 * O receives nrows*d values and lse nrows values, in the order of `rows`.
 * Returns 0, or -1 on a bad shape or row.
 */
int oracle_fwd_rows(const oracle_shape* s, const void* Q, const void* K, const void* V,
                    const void* Kd, const void* Vd, int64_t nrows, const int64_t* rows,
                    double* O, double* lse)
{
    if (!shape_ok(s)) return -1;
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t b = rows[3 * i], h = rows[3 * i + 1], t = rows[3 * i + 2];
        if (b < 0 || b >= s->B || h < 0 || h >= s->Hq || t < 0 || t >= s->T) return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(s->T + s->L + 1));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < nrows; ++i)
                row_forward(s, Q, K, V, Kd, Vd, rows[3 * i], rows[3 * i + 1], rows[3 * i + 2],
                            scores, O + i * s->d, lse + i);
            free(scores);
        }
    }
    return bad ? -1 : 0;
}

/*
 * Backward restricted to the query rows of one KV group at a set of tokens:
 * batch b, KV head kv, its G query heads h = kv*G + g, and the n distinct
 * tokens tok[0..n-1].  Every output holds exactly the contribution of those
 * rows:
 *   dQ  [G, n, d]         gradient rows of those queries (complete)
 *   dK, dV [T, d]         for every key, the sum over those rows that see it
 *   dKd, dVd [n*L, d]     the L depth rows of each selected token, in the order
 *                         of tok (complete: only that token's rows see them)
 *   O [G, n, d], lse [G, n]   the forward rows (by-products)
 * A row's contribution to dK, dV is scale*ds*Q and p*dO with ds = p (<dO,v> - D),
 * D = <dO, O>; both vanish when dO is zero at that row.  So when the upstream
 * gradient is zero at every other token of the group, dK and dV here are the
 * group's complete gradients.
 * dO has the storage code of the inputs.  Returns 0, or -1 on bad arguments.
 */
int oracle_bwd_tokens(const oracle_shape* s, int64_t b, int64_t kv, int64_t n,
                      const int64_t* tok, const void* Q, const void* K, const void* V,
                      const void* Kd, const void* Vd, const void* dO, double* dQ, double* dK,
                      double* dV, double* dKd, double* dVd, double* O, double* lse)
{
    if (!shape_ok(s) || b < 0 || b >= s->B || kv < 0 || kv >= s->Hk || n < 1) return -1;
    for (int64_t i = 0; i < n; ++i)
        if (tok[i] < 0 || tok[i] >= s->T) return -1;
    const int64_t G = s->Hq / s->Hk, L = s->L, d = s->d, l0 = first_slot(s);
    double* D = (double*)malloc(sizeof(double) * (size_t)(G * n));
    if (!D) return -1;
    int bad = 0;

    /* Step 1: forward rows, their log-sum-exp and D = <dO, O>. */
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(s->T + L + 1));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t i = 0; i < G * n; ++i) {
                const int64_t g = i / n, t = tok[i % n], h = kv * G + g;
                double* o = O + i * d;
                row_forward(s, Q, K, V, Kd, Vd, b, h, t, scores, o, lse + i);
                double acc = 0.0;
                const int64_t qo = q_off(s, b, h, t);
                for (int64_t e = 0; e < d; ++e) acc += elem(dO, s->dtype, qo + e) * o[e];
                D[i] = acc;
            }
            free(scores);
        }
    }
    if (bad) {
        free(D);
        return -1;
    }

    /* Step 2: per token, dQ of its G rows and the gradients of its own depth rows
     * (only that token's G query rows see them; slots before first_slot are not
     * visible and get zero gradient). */
    memset(dKd, 0, sizeof(double) * (size_t)(n * L * d));
    memset(dVd, 0, sizeof(double) * (size_t)(n * L * d));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t tt = 0; tt < n; ++tt) {
        const int64_t t = tok[tt];
        for (int64_t g = 0; g < G; ++g) {
            const int64_t h = kv * G + g, i = g * n + tt, qo = q_off(s, b, h, t);
            double* dq = dQ + i * d;
            for (int64_t e = 0; e < d; ++e) dq[e] = 0.0;
            for (int64_t j = 0; j <= last_key(s, t); ++j) {
                const int64_t ko = kv_off(s, b, kv, j);
                const double sc = s->scale * dot(s, Q, qo, K, ko);
                const double p = exp(sc - lse[i]);
                const double ds = p * (dot(s, dO, qo, V, ko) - D[i]);
                for (int64_t e = 0; e < d; ++e) dq[e] += s->scale * ds * elem(K, s->dtype, ko + e);
            }
            for (int64_t l = l0; l < L; ++l) {
                const int64_t ro = dep_off(s, b, kv, t * L + l);
                const double u = s->scale * dot(s, Q, qo, Kd, ro);
                const double q = exp(u - lse[i]);
                const double du = q * (dot(s, dO, qo, Vd, ro) - D[i]);
                double* dkd = dKd + (tt * L + l) * d;
                double* dvd = dVd + (tt * L + l) * d;
                for (int64_t e = 0; e < d; ++e) {
                    dq[e] += s->scale * du * elem(Kd, s->dtype, ro + e);
                    dkd[e] += s->scale * du * elem(Q, s->dtype, qo + e);
                    dvd[e] += q * elem(dO, s->dtype, qo + e);
                }
            }
        }
    }

    /* Step 3: per sequence key j, the sum over the selected rows that see it. */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < s->T; ++j) {
        const int64_t ko = kv_off(s, b, kv, j);
        double* dk = dK + j * d;
        double* dv = dV + j * d;
        for (int64_t e = 0; e < d; ++e) dk[e] = dv[e] = 0.0;
        for (int64_t tt = 0; tt < n; ++tt) {
            const int64_t t = tok[tt];
            if (j > last_key(s, t)) continue;
            for (int64_t g = 0; g < G; ++g) {
                const int64_t h = kv * G + g, i = g * n + tt, qo = q_off(s, b, h, t);
                const double sc = s->scale * dot(s, Q, qo, K, ko);
                const double p = exp(sc - lse[i]);
                const double ds = p * (dot(s, dO, qo, V, ko) - D[i]);
                for (int64_t e = 0; e < d; ++e) {
                    dk[e] += s->scale * ds * elem(Q, s->dtype, qo + e);
                    dv[e] += p * elem(dO, s->dtype, qo + e);
                }
            }
        }
    }
    free(D);
    return 0;
}

/* Threads the OpenMP runtime will use (reported beside CPU timings). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
