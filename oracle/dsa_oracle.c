/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DSA prefill hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker the GPU path is compared
 * against; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (one prompt chunk of n_q queries appended at cache position
 * `offset`; query i sits at absolute position p_i = offset + i):
 *
 *   1. Indexer score of every causal key (feedman.me page, per-component
 *      profile row "DSA indexer"; the formula itself is not printed on the
 *      pages, the reading used is a ReLU of each indexer head's dot product,
 *      weighted per head and summed):
 *          s[i][j] = sum_h w[i][h] * max(0, sum_d qidx[i][h][d] * kidx[j][d])
 *      for 0 <= j <= p_i, and -inf for p_i < j < ld.  Accumulated in fp64,
 *      rounded once to fp32; a zero score is written as +0.0.
 *
 *   2. Per-query top-k selection (same page, the paragraph on the work that
 *      is not a matmul: each query gathers the 2,048 keys it selected): if p_i + 1 <= k every causal key is kept; otherwise the keys
 *      are sorted by score descending, then by key index ascending (lower
 *      index wins a tie), and the first k are kept. The kept indices are
 *      written in ascending order and padded with -1 up to k.
 *
 *   3. Sparse attention over the kept keys (same page: the profile table's
 *      DSA sparse-attention core row; its hand-off paragraph gives each token
 *      a latent KV row 512 values wide): for each head h,
 *          l_j  = sm_scale * sum_{d < d_qk} q[i][h][d] * kv[j][d]
 *          o[c] = sum_j softmax(l)_j * kv[j][c]     for c < d_v
 *          lse  = log(sum_j exp(l_j))
 *      over the slots j of the row with 0 <= j <= p_i (other slots, such as
 *      the -1 padding, are ignored). A row with no valid slot gives o = 0 and
 *      lse = -inf. All arithmetic in fp64 (TensorFold issue #743, "Proposal:
 *      restore single-Mac GLM-5.3-Flash on the M3 Ultra": kernels that change
 *      the order of a reduction are validated against fp64 references).
 *
 * Inputs of dtype code 0 are bf16 bit patterns (uint16), widened exactly; code
 * 1 is fp32. Every function takes an optional list of query rows to compute
 * (rows == NULL means all n_q rows in order); outputs are compact, one entry
 * per listed row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_F32 1

static double oracle_load(const void *base, int dtype, int64_t pos) {
  if (dtype == ORACLE_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[pos]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[pos];
}

static int oracle_row(const int *rows, int r) { return rows ? rows[r] : r; }

/* Step 1: indexer scores. scores is [n_rows][ld]. Returns 0, or -1 on bad args. */
int oracle_indexer_scores(int n_q, int offset, int n_idx_heads, int d_idx, int idx_dtype,
                          const void *q_idx, const float *w, const void *k_idx,
                          float *scores, int64_t ld, const int *rows, int n_rows) {
  if (n_q < 0 || offset < 0 || n_idx_heads <= 0 || d_idx <= 0 || ld < (int64_t)offset + n_q)
    return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    const int i = oracle_row(rows, r);
    const int64_t p = (int64_t)offset + i;
    float *out = scores + (int64_t)r * ld;
    for (int64_t j = 0; j < ld; ++j) {
      if (j > p) {
        out[j] = -INFINITY;
        continue;
      }
      double s = 0.0;
      for (int h = 0; h < n_idx_heads; ++h) {
        double dot = 0.0;
        for (int d = 0; d < d_idx; ++d)
          dot += oracle_load(q_idx, idx_dtype, ((int64_t)i * n_idx_heads + h) * d_idx + d) *
                 oracle_load(k_idx, idx_dtype, j * d_idx + d);
        double relu = dot > 0.0 ? dot : 0.0;
        s += (double)w[(int64_t)i * n_idx_heads + h] * relu;
      }
      float f = (float)s;
      out[j] = (f == 0.0f) ? 0.0f : f; /* +0.0, never -0.0 */
    }
  }
  return 0;
}

typedef struct {
  float s;
  int32_t j;
} oracle_pair;

/* score descending, then key index ascending */
static int oracle_pair_cmp(const void *a, const void *b) {
  const oracle_pair *x = (const oracle_pair *)a, *y = (const oracle_pair *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int oracle_int_cmp(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* Step 2: top-k. scores is [n_rows][ld] (row r belongs to query rows[r]);
 * idx is [n_rows][top_k]. */
int oracle_topk_select(int n_q, int offset, int top_k, const float *scores, int64_t ld,
                       int32_t *idx, const int *rows, int n_rows) {
  if (n_q < 0 || offset < 0 || top_k <= 0 || ld < (int64_t)offset + n_q) return -1;
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    const int i = oracle_row(rows, r);
    const int64_t n = (int64_t)offset + i + 1; /* causal keys 0..p_i */
    const float *row = scores + (int64_t)r * ld;
    int32_t *out = idx + (int64_t)r * top_k;
    if (n <= top_k) {
      for (int64_t t = 0; t < top_k; ++t) out[t] = t < n ? (int32_t)t : -1;
      continue;
    }
    oracle_pair *pairs = (oracle_pair *)malloc((size_t)n * sizeof(oracle_pair));
    if (!pairs) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    for (int64_t j = 0; j < n; ++j) {
      pairs[j].s = row[j];
      pairs[j].j = (int32_t)j;
    }
    qsort(pairs, (size_t)n, sizeof(oracle_pair), oracle_pair_cmp);
    for (int t = 0; t < top_k; ++t) out[t] = pairs[t].j;
    qsort(out, (size_t)top_k, sizeof(int32_t), oracle_int_cmp);
    free(pairs);
  }
  return status;
}

/* Step 3: sparse attention. idx is [n_rows][top_k] (row r belongs to query
 * rows[r]); out is [n_rows][n_heads][d_v]; lse is [n_rows][n_heads] or NULL. */
int oracle_sparse_mla(int n_q, int offset, int n_heads, int d_qk, int d_v, double sm_scale,
                      int act_dtype, const void *q, const void *kv, const int32_t *idx,
                      int top_k, double *out, double *lse, const int *rows, int n_rows) {
  if (n_q < 0 || offset < 0 || n_heads <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk ||
      top_k <= 0)
    return -1;
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    const int i = oracle_row(rows, r);
    const int64_t p = (int64_t)offset + i;
    const int32_t *sel = idx + (int64_t)r * top_k;
    double *logit = (double *)malloc((size_t)top_k * sizeof(double));
    if (!logit) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    for (int h = 0; h < n_heads; ++h) {
      const int64_t qbase = ((int64_t)i * n_heads + h) * d_qk;
      double *o = out + ((int64_t)r * n_heads + h) * d_v;
      double m = -INFINITY;
      for (int t = 0; t < top_k; ++t) {
        const int64_t j = sel[t];
        if (j < 0 || j > p) continue;
        double dot = 0.0;
        for (int d = 0; d < d_qk; ++d)
          dot += oracle_load(q, act_dtype, qbase + d) * oracle_load(kv, act_dtype, j * d_qk + d);
        logit[t] = sm_scale * dot;
        if (logit[t] > m) m = logit[t];
      }
      for (int c = 0; c < d_v; ++c) o[c] = 0.0;
      if (m == -INFINITY) { /* no valid slot */
        if (lse) lse[(int64_t)r * n_heads + h] = -INFINITY;
        continue;
      }
      double l = 0.0;
      for (int t = 0; t < top_k; ++t) {
        const int64_t j = sel[t];
        if (j < 0 || j > p) continue;
        const double e = exp(logit[t] - m);
        l += e;
        for (int c = 0; c < d_v; ++c) o[c] += e * oracle_load(kv, act_dtype, j * d_qk + c);
      }
      for (int c = 0; c < d_v; ++c) o[c] /= l;
      if (lse) lse[(int64_t)r * n_heads + h] = m + log(l);
    }
    free(logit);
  }
  return status;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the parallel loops that follow (a timing knob; results do not
 * depend on it: every row is computed by one thread in a fixed order). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
