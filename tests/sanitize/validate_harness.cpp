// validate_harness.cpp -- host-only driver of the C ABI's argument checks
// (validate.cpp) and of the matrix-core self-test's reference values
// (selftest_ref.h), built with AddressSanitizer and UndefinedBehaviorSanitizer
// by the CPU tests. Exits non-zero on the first failed expectation or any
// sanitizer report.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "selftest_ref.h"
#include "validate.h"

static int g_fails = 0;
#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++g_fails;                                                      \
    }                                                                 \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t F = 1u << 20;  // an aligned address that is never dereferenced

static dsa_dims dims() {
  dsa_dims d;
  d.n_q = 16;
  d.offset = 100;
  d.n_heads = 64;
  d.d_latent = 512;
  d.d_rope = 64;
  d.n_idx_heads = 4;
  d.d_idx = 128;
  d.top_k = 2048;
  d.sm_scale = 1.0f / 24.0f;
  d.act_dtype = DSA_BF16;
  d.idx_dtype = DSA_BF16;
  return d;
}

static void indexer_checks() {
  dsa::IndexerArgs a{};
  dsa_dims d = dims();
  EXPECT(dsa::check_indexer(&d, P(F), (float*)P(F), P(F), (float*)P(F), 116, &a) == DSA_OK);
  EXPECT(a.n_q == 16 && a.ld == 116 && a.bf16);
  EXPECT(dsa::check_indexer(nullptr, P(F), (float*)P(F), P(F), (float*)P(F), 116, &a) == DSA_ERR_NULL);
  EXPECT(dsa::check_indexer(&d, P(F), (float*)P(F), P(F), (float*)P(F), 115, &a) == DSA_ERR_SHAPE);
  EXPECT(dsa::check_indexer(&d, P(F), nullptr, P(F), (float*)P(F), 116, &a) == DSA_ERR_NULL);
  EXPECT(dsa::check_indexer(&d, P(F + 4), (float*)P(F), P(F), (float*)P(F), 116, &a) == DSA_ERR_ALIGN);
  d.offset = 0x7fffffff - 5;
  EXPECT(dsa::check_indexer(&d, P(F), (float*)P(F), P(F), (float*)P(F), (int64_t)1 << 32, &a) == DSA_ERR_SHAPE);
  d = dims();
  d.idx_dtype = 9;
  EXPECT(dsa::check_indexer(&d, P(F), (float*)P(F), P(F), (float*)P(F), 116, &a) == DSA_ERR_DTYPE);
  d = dims();
  d.n_idx_heads = 3;
  d.d_idx = 4096;
  EXPECT(dsa::check_indexer(&d, P(F), (float*)P(F), P(F), (float*)P(F), 116, &a) == DSA_ERR_UNSUPPORTED);
  d = dims();
  d.n_q = 0;
  EXPECT(dsa::check_indexer(&d, nullptr, nullptr, nullptr, nullptr, 100, &a) == DSA_OK);
  // extreme values must not overflow (UBSan watches the arithmetic)
  d = dims();
  d.n_q = 0x7fffffff;
  d.offset = 0;
  d.n_idx_heads = 0x7fffffff;
  d.d_idx = 0x7fffffff;
  EXPECT(dsa::check_indexer(&d, P(F), (float*)P(F), P(F), (float*)P(F), (int64_t)1 << 40, &a) == DSA_ERR_UNSUPPORTED);
}

static void topk_checks() {
  dsa::TopkArgs a{};
  dsa_dims d = dims();
  EXPECT(dsa::check_topk(&d, (float*)P(F), 116, (int32_t*)P(F), 0, &a) == DSA_OK);
  EXPECT(dsa::check_topk(&d, (float*)P(F), 115, (int32_t*)P(F), 0, &a) == DSA_ERR_SHAPE);
  EXPECT(dsa::check_topk(&d, nullptr, 116, (int32_t*)P(F), 0, &a) == DSA_ERR_NULL);
  EXPECT(dsa::check_topk(&d, (float*)P(F), 116, (int32_t*)P(F + 8), 0, &a) == DSA_ERR_ALIGN);
  d.top_k = 0;
  EXPECT(dsa::check_topk(&d, (float*)P(F), 116, (int32_t*)P(F), 0, &a) == DSA_ERR_SHAPE);
  d.top_k = (1 << 20) + 1;
  EXPECT(dsa::check_topk(&d, (float*)P(F), 116, (int32_t*)P(F), 0, &a) == DSA_ERR_SHAPE);
}

static void mla_checks() {
  dsa::MlaArgs a{};
  dsa_dims d = dims();
  EXPECT(dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), nullptr, &a) == DSA_OK);
  EXPECT(dsa::mla_fast_path(a));
  EXPECT(dsa::check_mla(&d, P(F), nullptr, (int32_t*)P(F), (float*)P(F), nullptr, &a) == DSA_ERR_NULL);
  EXPECT(dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), (float*)P(F + 4), &a) == DSA_ERR_ALIGN);
  d.sm_scale = 1.0f / 0.0f;
  EXPECT(dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), nullptr, &a) == DSA_ERR_SHAPE);
  d = dims();
  d.n_heads = 8;
  d.d_latent = 4000;
  EXPECT(dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), nullptr, &a) == DSA_ERR_UNSUPPORTED);
  d = dims();
  d.top_k = 130;  // not a multiple of 4: the plain kernel
  EXPECT(dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), nullptr, &a) == DSA_OK);
  EXPECT(!dsa::mla_fast_path(a));
  // a cache of 4 GiB or more leaves the fast path (32-bit row offsets)
  d = dims();
  d.offset = (int32_t)(((int64_t)1 << 32) / 1152);
  EXPECT(dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), nullptr, &a) == DSA_OK);
  EXPECT(!dsa::mla_fast_path(a));
}

static void decode_split_checks() {
  // every split is whole tiles, covers the row, and the workspace matches
  for (int n_q = 1; n_q <= 300; n_q += 7) {
    for (int top_k : {4, 32, 100, 128, 132, 2048, 4096, 4100}) {
      dsa_dims d = dims();
      d.n_q = n_q;
      d.top_k = top_k;
      dsa::MlaArgs a{};
      if (dsa::check_mla(&d, P(F), P(F), (int32_t*)P(F), (float*)P(F), nullptr, &a) != DSA_OK) continue;
      const dsa::MlaSplit sp = dsa::mla_decode_split(a);
      EXPECT(sp.splits >= 1);
      if (sp.splits > 1) {
        EXPECT(sp.split_slots % dsa::kDecodeTile == 0);
        EXPECT((int64_t)sp.splits * sp.split_slots >= top_k);
        EXPECT((int64_t)(sp.splits - 1) * sp.split_slots < top_k);  // no empty trailing split
        EXPECT(dsa::mla_decode_workspace_bytes(a) == (size_t)sp.splits * n_q * 64 * 513 * 4);
      } else {
        EXPECT(dsa::mla_decode_workspace_bytes(a) == 0);
      }
    }
  }
  EXPECT(dsa::check_workspace(nullptr, 0, 0) == DSA_OK);
  EXPECT(dsa::check_workspace(nullptr, 0, 64) == DSA_ERR_WORKSPACE);
  EXPECT(dsa::check_workspace(P(F), 63, 64) == DSA_ERR_WORKSPACE);
  EXPECT(dsa::check_workspace(P(F + 4), 64, 64) == DSA_ERR_ALIGN);
}

static void append_checks() {
  dsa_dims d = dims();
  const uintptr_t cache = 4 * F;
  const uintptr_t dst = cache + 100 * 1152;
  EXPECT(dsa::check_append(&d, P(F), P(F), P(cache), P(8 * F)) == DSA_OK);
  EXPECT(dsa::check_append(&d, P(dst), P(F), P(cache), P(8 * F)) == DSA_OK);          // in place
  EXPECT(dsa::check_append(&d, P(dst + 1152), P(F), P(cache), P(8 * F)) == DSA_ERR_SHAPE);  // partial overlap
  EXPECT(dsa::check_append(&d, nullptr, P(F), P(cache), P(8 * F)) == DSA_ERR_NULL);
  EXPECT(dsa::check_append(&d, P(F), P(F + 4), P(cache), P(8 * F)) == DSA_ERR_ALIGN);
}

// The self-test's comparison must reject the layouts a kernel could get
// wrong: a transposed result or operand, and swapped k-slices of an operand.
static void selftest_power_checks() {
  using namespace dsa::selftest;
  std::vector<float> e(kOutFloats);
  expected(e.data());
  EXPECT(count_mismatches(e.data()) == 0);
  int off = 0;
  for (int c = 0; c < 3; ++c) {
    int M, N, K;
    dims_of(c, &M, &N, &K);
    // transposed result (M == N in every case)
    std::vector<float> t = e;
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) t[off + m * N + n] = e[off + n * N + m];
    EXPECT(count_mismatches(t.data()) > 0);
    // A's k-slices swapped (lane halves / quarters exchanged)
    std::vector<float> s = e;
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) {
        int acc = 0;
        for (int k = 0; k < K; ++k) acc += a_val(c, m, k ^ 8) * b_val(c, k, n);
        s[off + m * N + n] = (float)acc;
      }
    EXPECT(count_mismatches(s.data()) > 0);
    // B transposed within its square blocks: B'[k][n] = B[n][k] for k, n < N
    std::vector<float> b = e;
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) {
        int acc = 0;
        for (int k = 0; k < K; ++k) acc += a_val(c, m, k) * (k < N ? b_val(c, n, k) : b_val(c, k, n));
        b[off + m * N + n] = (float)acc;
      }
    EXPECT(count_mismatches(b.data()) > 0);
    off += M * N;
  }
}

int main() {
  indexer_checks();
  topk_checks();
  mla_checks();
  decode_split_checks();
  append_checks();
  selftest_power_checks();
  if (g_fails) fprintf(stderr, "%d expectation(s) failed\n", g_fails);
  else printf("validate harness: ok\n");
  return g_fails ? 1 : 0;
}
