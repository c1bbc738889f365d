/* oracle_harness.c -- drives the CPU oracle (oracle/dsa_oracle.c) on small
 * random and edge-case inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by the CPU tests). The values are checked
 * by the oracle's pins elsewhere; this run looks for memory and undefined-
 * behaviour errors, plus two invariants (selected counts, finite outputs). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_indexer_scores(int n_q, int offset, int n_idx_heads, int d_idx, int idx_dtype, const void *q_idx,
                          const float *w, const void *k_idx, float *scores, int64_t ld, const int *rows, int n_rows);
int oracle_topk_select(int n_q, int offset, int top_k, const float *scores, int64_t ld, int32_t *idx,
                       const int *rows, int n_rows);
int oracle_sparse_mla(int n_q, int offset, int n_heads, int d_qk, int d_v, double sm_scale, int act_dtype,
                      const void *q, const void *kv, const int32_t *idx, int top_k, double *out, double *lse,
                      const int *rows, int n_rows);

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state >> 8;
}

static int run_case(int n_q, int offset, int H_I, int D_I, int H, int d_qk, int d_v, int k, int with_rows) {
  const int t_ctx = offset + n_q;
  const int64_t ld = t_ctx + 3;
  float *qidx = malloc(sizeof(float) * (size_t)n_q * H_I * D_I);
  float *kidx = malloc(sizeof(float) * (size_t)t_ctx * D_I);
  float *w = malloc(sizeof(float) * (size_t)n_q * H_I);
  float *q = malloc(sizeof(float) * (size_t)n_q * H * d_qk);
  float *kv = malloc(sizeof(float) * (size_t)t_ctx * d_qk);
  for (int e = 0; e < n_q * H_I * D_I; ++e) qidx[e] = (float)((int)(rnd() % 7) - 3);
  for (int e = 0; e < t_ctx * D_I; ++e) kidx[e] = (float)((int)(rnd() % 7) - 3);
  for (int e = 0; e < n_q * H_I; ++e) w[e] = (float)(1 + rnd() % 2);
  for (int e = 0; e < n_q * H * d_qk; ++e) q[e] = (float)((int)(rnd() % 2001) - 1000) / 1000.0f;
  for (int e = 0; e < t_ctx * d_qk; ++e) kv[e] = (float)((int)(rnd() % 2001) - 1000) / 1000.0f;
  int n_rows = n_q;
  int *rows = NULL;
  if (with_rows) { /* every other row, in reverse */
    n_rows = (n_q + 1) / 2;
    rows = malloc(sizeof(int) * (size_t)n_rows);
    for (int r = 0; r < n_rows; ++r) rows[r] = n_q - 1 - 2 * r;
  }
  float *scores = malloc(sizeof(float) * (size_t)n_rows * ld);
  int32_t *idx = malloc(sizeof(int32_t) * (size_t)n_rows * k);
  double *out = malloc(sizeof(double) * (size_t)n_rows * H * d_v);
  double *lse = malloc(sizeof(double) * (size_t)n_rows * H);
  int bad = 0;
  bad |= oracle_indexer_scores(n_q, offset, H_I, D_I, 1, qidx, w, kidx, scores, ld, rows, n_rows) != 0;
  bad |= oracle_topk_select(n_q, offset, k, scores, ld, idx, rows, n_rows) != 0;
  bad |= oracle_sparse_mla(n_q, offset, H, d_qk, d_v, 0.125, 1, q, kv, idx, k, out, lse, rows, n_rows) != 0;
  for (int r = 0; r < n_rows && !bad; ++r) {
    const int i = rows ? rows[r] : r;
    int cnt = 0;
    for (int t = 0; t < k; ++t) cnt += idx[(int64_t)r * k + t] >= 0;
    const int n = offset + i + 1;
    if (cnt != (n < k ? n : k)) bad = 1;
    for (int h = 0; h < H; ++h)
      if (!isfinite(lse[(int64_t)r * H + h])) bad = 1;
  }
  free(qidx); free(kidx); free(w); free(q); free(kv); free(rows); free(scores); free(idx); free(out); free(lse);
  if (bad) fprintf(stderr, "oracle case n_q=%d offset=%d k=%d failed\n", n_q, offset, k);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run_case(1, 0, 1, 1, 1, 1, 1, 1, 0);       /* single key */
  bad |= run_case(9, 0, 2, 8, 2, 12, 8, 16, 0);     /* every row shorter than k */
  bad |= run_case(17, 40, 2, 8, 3, 20, 16, 8, 0);   /* select with ties */
  bad |= run_case(33, 70, 4, 16, 4, 24, 16, 20, 1); /* a row subset */
  /* argument errors are reported, not acted on */
  float s = 0.0f;
  int32_t ix = 0;
  bad |= oracle_topk_select(-1, 0, 4, &s, 1, &ix, NULL, 0) != -1;
  bad |= oracle_indexer_scores(1, 0, 1, 1, 1, &s, &s, &s, &s, 0, NULL, 1) != -1;
  if (!bad) printf("oracle harness: ok\n");
  return bad;
}
