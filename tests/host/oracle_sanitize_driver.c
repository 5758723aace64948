/* Host driver for the sanitizer test of the oracle (test infrastructure):
 * runs every oracle entry point on seeded random ragged inputs (empty
 * sequences, qo > kv, sampled rows) so that an out-of-bounds index or an
 * undefined operation in it is reported. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_prefill(const void *q, const void *k, const void *v, int dtype,
                   const int32_t *qo_indptr, const int32_t *kv_indptr, int batch,
                   int num_heads, int dqk, int dvo, int causal, double sm_scale,
                   const int64_t *rows, int64_t n_rows, double *out, double *lse);
int oracle_absorbed(const void *q, const void *kv, int dtype, const int32_t *qo_indptr,
                    const int32_t *kv_indptr, int batch, int num_heads, int dqk, int dvo,
                    int causal, double sm_scale, const int64_t *rows, int64_t n_rows,
                    double *out, double *lse);
int oracle_merge(const void *o_a, const void *lse_a, const void *o_b, const void *lse_b,
                 int o_dtype, int lse_dtype, int64_t rows, int dim, double *o, double *lse);
int oracle_decompress(const void *c_kv, const void *k_rope, const void *w_uk, const void *w_uv,
                      int dtype, int64_t num_tokens, int num_heads, int dlat, int dnope,
                      int drope, int dvo, const int64_t *rows, int64_t n_rows,
                      double *k_out, double *v_out);

static uint64_t state = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in [-1, 1) */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / (double)(1ull << 52) - 1.0;
}
static double *alloc_rand(int64_t n) {
    double *p = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

int main(void) {
    const int fp64 = 2;
    int calls = 0;
    for (int trial = 0; trial < 40; ++trial) {
        const int batch = 1 + (int)(state % 4);
        int32_t qo[5] = {0}, kv[5] = {0};
        for (int b = 0; b < batch; ++b) {
            rnd();
            qo[b + 1] = qo[b] + (int)(state % 9);
            rnd();
            kv[b + 1] = kv[b] + (int)(state % 13);
        }
        const int h = 1 + trial % 3, dqk = 8, dvo = 4;
        const int64_t tq = qo[batch], tk = kv[batch];
        const int64_t out_rows = tq > 3 ? tq : 3;   /* all rows, or the 3 sampled */
        double *q = alloc_rand(tq * h * dqk), *k = alloc_rand(tk * h * dqk),
               *v = alloc_rand(tk * h * dvo), *out = alloc_rand(out_rows * h * dvo),
               *lse = alloc_rand(out_rows * h);
        int64_t rows[3] = {0, tq > 1 ? tq - 1 : 0, tq / 2};
        for (int causal = 0; causal < 2; ++causal) {
            calls += oracle_prefill(q, k, v, fp64, qo, kv, batch, h, dqk, dvo, causal, 0.3, NULL,
                                    tq, out, lse) == 0;
            if (tq > 0)
                calls += oracle_prefill(q, k, v, fp64, qo, kv, batch, h, dqk, dvo, causal, 0.3,
                                        rows, 3, out, lse) == 0;
            /* absorbed: one shared row of dqk per key, value = its first dvo dims */
            calls += oracle_absorbed(q, k, fp64, qo, kv, batch, h, dqk, dvo, causal, 0.3, NULL,
                                     tq, out, lse) == 0;
        }
        calls += oracle_merge(out, lse, out, lse, fp64, fp64, tq * h / (h > 0 ? h : 1), dvo,
                              out, lse) == 0;
        double *c = alloc_rand(tk * 16), *r = alloc_rand(tk * 4), *wk = alloc_rand(16 * h * 8),
               *wv = alloc_rand(16 * h * 8), *ko = alloc_rand(tk * h * 12),
               *vo = alloc_rand(tk * h * 8);
        calls += oracle_decompress(c, r, wk, wv, fp64, tk, h, 16, 8, 4, 8, NULL, tk, ko, vo) == 0;
        free(q); free(k); free(v); free(out); free(lse);
        free(c); free(r); free(wk); free(wv); free(ko); free(vo);
    }
    printf("oracle sanitize driver: %d calls returned 0\n", calls);
    return 0;
}
