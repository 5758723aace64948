/*
 * oracle.c -- plain, slow, fp64 CPU reference for MLA ragged prefill,
 * merge_state and MLA KV decompression.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header or constant with the HIP library and must never sit on the
 * product path.
 *
 * What it follows:
 *  - "vllm.v1.attention.backends.mla.prefill.flashinfer", finalize_attention_metadata
 *    and run_prefill_new_tokens / run_prefill_context_chunk: attention over a
 *    ragged batch indexed by qo_indptr / kv_indptr, NHD layout, one causal
 *    pass over the new tokens (kv_indptr equal to qo_indptr) and one
 *    non-causal pass per context chunk; each pass returns O and the
 *    log-sum-exp, LSE laid out [tokens, heads].
 *  - "[DeepseekR1] How ragged prefill manage kv_cache?" (sglang issue 3849):
 *    query/key head dim 192, value/output head dim 128; the cache holds a
 *    512-dim latent plus 64 RoPE dims; ragged prefill returns the LSE.
 *  - "[KVCache] PagedKVCache refactor, FlashInfer JIT and MLA integration"
 *    (apache/tvm PR 17674): the softmax scale is always passed explicitly.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - LSE is the natural-log normaliser of the SCALED logits.
 *  - Causal masking is bottom-right aligned: query row i of a sequence with
 *    qo_len queries and kv_len keys sees keys j < kv_len - qo_len + i + 1.
 *  - A row that sees no key gets O = 0 and LSE = -inf.
 *  - merge of two states with LSE a, b: lse = log(e^a + e^b),
 *    o = e^(a-lse) o_a + e^(b-lse) o_b; a side with LSE = -inf has weight 0;
 *    both -inf gives o = 0, lse = -inf.
 *  - Decompression: K_nope[t,h,d] = sum_c c_kv[t,c] W_UK[c, h*128+d],
 *    V[t,h,d] = sum_c c_kv[t,c] W_UV[c, h*128+d], K = [K_nope | k_rope[t]].
 *
 * Every floating-point step is fp64; inputs in bf16 or fp32 are widened
 * exactly. No blocking, fusion or reordering beyond the definitions: two
 * passes per row (scores; then max, exponentials, sum and the weighted sum
 * of V rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_FP32 1
#define ORACLE_FP64 2

/* Widen element `idx` of an array of the given dtype to double. */
static double load_elem(const void *base, int dtype, int64_t idx) {
    if (dtype == ORACLE_BF16) {
        uint16_t h = ((const uint16_t *)base)[idx];
        uint32_t bits = ((uint32_t)h) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_FP32) return (double)((const float *)base)[idx];
    return ((const double *)base)[idx];
}

/* Sequence that owns row t: the b with indptr[b] <= t < indptr[b+1]. */
static int owner(const int32_t *indptr, int batch, int64_t t) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if ((int64_t)indptr[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/*
 * Number of keys query row i may see: all kv_len keys when not causal; with
 * bottom-right causal alignment, keys j < kv_len - qo_len + i + 1 (never
 * below 0, never above kv_len).
 */
static int64_t visible_keys(int64_t i, int64_t qo_len, int64_t kv_len, int causal) {
    if (!causal) return kv_len;
    int64_t n = kv_len - qo_len + i + 1;
    if (n < 0) n = 0;
    if (n > kv_len) n = kv_len;
    return n;
}

/*
 * Attention for a list of query rows.
 *   q [Tq, H, dqk], k [Tk, H, dqk], v [Tk, H, dvo] of dtype `dtype`.
 *   rows: query token indices to compute (n_rows of them), or NULL for all Tq.
 *   out [n_rows, H, dvo] and lse [n_rows, H] in fp64.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_prefill(const void *q, const void *k, const void *v, int dtype,
                   const int32_t *qo_indptr, const int32_t *kv_indptr, int batch,
                   int num_heads, int dqk, int dvo, int causal, double sm_scale,
                   const int64_t *rows, int64_t n_rows, double *out, double *lse) {
    if (batch < 1 || num_heads < 1 || dqk < 1 || dvo < 1) return -1;
    if (rows == NULL) n_rows = qo_indptr[batch];
    int64_t max_kv = 0;
    for (int b = 0; b < batch; ++b) {
        int64_t n = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        if (n > max_kv) max_kv = n;
    }
    int failed = 0;
#pragma omp parallel reduction(|:failed)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_kv > 0 ? max_kv : 1));
        if (s == NULL) failed = 1;
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < n_rows; ++r) {
            for (int h = 0; h < num_heads; ++h) {
                if (s == NULL) continue;
                int64_t t = rows ? rows[r] : r;
                int b = owner(qo_indptr, batch, t);
                int64_t qs = qo_indptr[b], ks = kv_indptr[b];
                int64_t qo_len = (int64_t)qo_indptr[b + 1] - qs;
                int64_t kv_len = (int64_t)kv_indptr[b + 1] - ks;
                int64_t i = t - qs;
                int64_t nv = visible_keys(i, qo_len, kv_len, causal);
                double *o_row = out + ((size_t)r * num_heads + h) * dvo;
                double *lse_out = lse + (size_t)r * num_heads + h;
                if (nv == 0) {
                    for (int d = 0; d < dvo; ++d) o_row[d] = 0.0;
                    *lse_out = -INFINITY;
                    continue;
                }
                /* pass 1: scaled scores s_j = sm_scale * <q_t, k_j> */
                int64_t qoff = ((int64_t)t * num_heads + h) * dqk;
                for (int64_t j = 0; j < nv; ++j) {
                    int64_t koff = ((ks + j) * num_heads + h) * dqk;
                    double dot = 0.0;
                    for (int d = 0; d < dqk; ++d)
                        dot += load_elem(q, dtype, qoff + d) * load_elem(k, dtype, koff + d);
                    s[j] = sm_scale * dot;
                }
                /* pass 2: m, l = sum exp(s - m), LSE = m + ln l, O = sum p_j v_j / l */
                double m = s[0];
                for (int64_t j = 1; j < nv; ++j) if (s[j] > m) m = s[j];
                double l = 0.0;
                for (int64_t j = 0; j < nv; ++j) { s[j] = exp(s[j] - m); l += s[j]; }
                *lse_out = m + log(l);
                for (int d = 0; d < dvo; ++d) o_row[d] = 0.0;
                for (int64_t j = 0; j < nv; ++j) {
                    double w = s[j] / l;
                    int64_t voff = ((ks + j) * num_heads + h) * dvo;
                    for (int d = 0; d < dvo; ++d) o_row[d] += w * load_elem(v, dtype, voff + d);
                }
            }
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/*
 * Weight-absorbed MLA attention over the latent cache (multi-query: one
 * shared key/value row per token). The query of head h is the 576-dim
 * absorbed query [q_nope W_UK_h | q_rope]; the key of token j is its cache
 * row kv[j] = [c_kv | k_rope] (576 dims), the value is the first dvo (512)
 * dims of the same row (the latent), and the output stays in the latent
 * space ("[DeepseekR1] How ragged prefill manage kv_cache?", sglang issue
 * 3849: the absorbed path, forward_absorb, that attends the latent cache
 * directly). Same visible-key rule, scaling and LSE as oracle_prefill.
 *   q [Tq, H, dqk] and kv [Tk, dqk] of dtype `dtype`; dvo <= dqk.
 *   rows: query token indices (n_rows of them), or NULL for all Tq.
 *   out [n_rows, H, dvo] and lse [n_rows, H] in fp64.
 */
int oracle_absorbed(const void *q, const void *kv, int dtype, const int32_t *qo_indptr,
                    const int32_t *kv_indptr, int batch, int num_heads, int dqk, int dvo,
                    int causal, double sm_scale, const int64_t *rows, int64_t n_rows,
                    double *out, double *lse) {
    if (batch < 1 || num_heads < 1 || dqk < 1 || dvo < 1 || dvo > dqk) return -1;
    if (rows == NULL) n_rows = qo_indptr[batch];
    int64_t max_kv = 0;
    for (int b = 0; b < batch; ++b) {
        int64_t n = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
        if (n > max_kv) max_kv = n;
    }
    int failed = 0;
#pragma omp parallel reduction(|:failed)
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)(max_kv > 0 ? max_kv : 1));
        if (sc == NULL) failed = 1;
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < n_rows; ++r) {
            for (int h = 0; h < num_heads; ++h) {
                if (sc == NULL) continue;
                int64_t t = rows ? rows[r] : r;
                int b = owner(qo_indptr, batch, t);
                int64_t qs = qo_indptr[b], ks = kv_indptr[b];
                int64_t qo_len = (int64_t)qo_indptr[b + 1] - qs;
                int64_t kv_len = (int64_t)kv_indptr[b + 1] - ks;
                int64_t nv = visible_keys(t - qs, qo_len, kv_len, causal);
                double *o_row = out + ((size_t)r * num_heads + h) * dvo;
                double *lse_out = lse + (size_t)r * num_heads + h;
                if (nv == 0) {
                    for (int d = 0; d < dvo; ++d) o_row[d] = 0.0;
                    *lse_out = -INFINITY;
                    continue;
                }
                /* pass 1: scaled scores against the shared cache rows */
                int64_t q_at = ((int64_t)t * num_heads + h) * dqk;
                for (int64_t j = 0; j < nv; ++j) {
                    int64_t row_at = (ks + j) * dqk;
                    double acc = 0.0;
                    for (int d = 0; d < dqk; ++d)
                        acc += load_elem(q, dtype, q_at + d) * load_elem(kv, dtype, row_at + d);
                    sc[j] = sm_scale * acc;
                }
                /* pass 2: softmax weights, LSE, weighted sum of the latent parts */
                double top = sc[0];
                for (int64_t j = 1; j < nv; ++j) if (sc[j] > top) top = sc[j];
                double den = 0.0;
                for (int64_t j = 0; j < nv; ++j) { sc[j] = exp(sc[j] - top); den += sc[j]; }
                *lse_out = top + log(den);
                for (int d = 0; d < dvo; ++d) o_row[d] = 0.0;
                for (int64_t j = 0; j < nv; ++j) {
                    double w = sc[j] / den;
                    int64_t latent_at = (ks + j) * dqk;
                    for (int d = 0; d < dvo; ++d) o_row[d] += w * load_elem(kv, dtype, latent_at + d);
                }
            }
        }
        free(sc);
    }
    return failed ? -1 : 0;
}

/*
 * Merge two attention states over disjoint key sets.
 *   o_a, o_b [rows, dim] of dtype o_dtype; lse_a, lse_b [rows] of dtype lse_dtype.
 *   o [rows, dim], lse [rows] in fp64.
 */
int oracle_merge(const void *o_a, const void *lse_a, const void *o_b, const void *lse_b,
                 int o_dtype, int lse_dtype, int64_t rows, int dim, double *o, double *lse) {
    if (rows < 0 || dim < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double a = load_elem(lse_a, lse_dtype, r);
        double b = load_elem(lse_b, lse_dtype, r);
        double mx = a > b ? a : b;
        double *o_row = o + (size_t)r * dim;
        if (mx == -INFINITY) {
            for (int d = 0; d < dim; ++d) o_row[d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double ea = exp(a - mx), eb = exp(b - mx);     /* exp(-inf) = 0 */
        double out_lse = mx + log(ea + eb);
        double wa = exp(a - out_lse), wb = exp(b - out_lse);
        for (int d = 0; d < dim; ++d) {
            double xa = wa == 0.0 ? 0.0 : wa * load_elem(o_a, o_dtype, r * (int64_t)dim + d);
            double xb = wb == 0.0 ? 0.0 : wb * load_elem(o_b, o_dtype, r * (int64_t)dim + d);
            o_row[d] = xa + xb;
        }
        lse[r] = out_lse;
    }
    return 0;
}

/*
 * Decompress the latent cache for a list of tokens.
 *   c_kv [T, dlat], k_rope [T, drope], w_uk [dlat, H*dnope], w_uv [dlat, H*dvo],
 *   all of dtype `dtype`.
 *   rows: token indices (n_rows), or NULL for all T (then n_rows = T).
 *   k_out [n_rows, H, dnope+drope], v_out [n_rows, H, dvo] in fp64.
 */
int oracle_decompress(const void *c_kv, const void *k_rope, const void *w_uk, const void *w_uv,
                      int dtype, int64_t num_tokens, int num_heads, int dlat, int dnope,
                      int drope, int dvo, const int64_t *rows, int64_t n_rows,
                      double *k_out, double *v_out) {
    if (num_heads < 1 || dlat < 1) return -1;
    if (rows == NULL) n_rows = num_tokens;
    int dqk = dnope + drope;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int h = 0; h < num_heads; ++h) {
            int64_t t = rows ? rows[r] : r;
            double *k_row = k_out + ((size_t)r * num_heads + h) * dqk;
            double *v_row = v_out + ((size_t)r * num_heads + h) * dvo;
            for (int d = 0; d < dnope; ++d) {
                double acc = 0.0;
                for (int c = 0; c < dlat; ++c)
                    acc += load_elem(c_kv, dtype, t * dlat + c) *
                           load_elem(w_uk, dtype, (int64_t)c * num_heads * dnope + (int64_t)h * dnope + d);
                k_row[d] = acc;
            }
            for (int d = 0; d < drope; ++d)
                k_row[dnope + d] = load_elem(k_rope, dtype, t * drope + d);
            for (int d = 0; d < dvo; ++d) {
                double acc = 0.0;
                for (int c = 0; c < dlat; ++c)
                    acc += load_elem(c_kv, dtype, t * dlat + c) *
                           load_elem(w_uv, dtype, (int64_t)c * num_heads * dvo + (int64_t)h * dvo + d);
                v_row[d] = acc;
            }
        }
    }
    return 0;
}

/* Threads the oracle will use (OpenMP), for reporting. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
