// selftest_ref.h -- operands and expected results of the matrix-core layout
// self-test (the load-time check that a kernel's operand and result layouts
// are the ones it assumes; TensorFold issue #743, "Proposal: restore
// single-Mac GLM-5.3-Flash on the M3 Ultra", asks for such a check, one that
// must catch a transposed operand).
//
// Three products of small integers (exact in bf16 and in fp32 sums), one per
// MFMA form and operand path the fast kernels use:
//   case 0: 16x16x32 bf16, A and B from registers       (attention Q K^T)
//   case 1: 32x32x16 bf16, A and B from registers       (indexer)
//   case 2: 16x16x32 bf16, B read transposed from LDS   (attention P V)
// The operand values are shared by the device kernel and the host check; the
// expected products are computed on the host by plain loops.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define DSA_HD __host__ __device__
#else
#define DSA_HD
#endif

namespace dsa {
namespace selftest {

constexpr int kCase0 = 16 * 16;  // C[16][16]
constexpr int kCase1 = 32 * 32;  // C[32][32]
constexpr int kCase2 = 16 * 16;  // C[16][16]
constexpr int kOutFloats = kCase0 + kCase1 + kCase2;

// Operands: A[m][k] and B[k][n], values in [-3, 3] (A) and [-2, 2] (B),
// neither symmetric nor periodic in a way a transposition or a swapped
// k-slice would preserve.
DSA_HD inline int a_val(int c, int m, int k) { return ((3 * m + 5 * k + 7 * c + 1) % 7) - 3; }
DSA_HD inline int b_val(int c, int k, int n) { return ((2 * k + 3 * n + 3 * c + 1 + (k * n) % 3) % 5) - 2; }

inline void dims_of(int c, int* M, int* N, int* K) {
  *M = c == 1 ? 32 : 16;
  *N = c == 1 ? 32 : 16;
  *K = c == 1 ? 16 : 32;
}

// Expected C[m][n] = sum_k A[m][k] B[k][n] of every case, row-major, packed
// one case after another (kOutFloats values).
inline void expected(float* out) {
  int off = 0;
  for (int c = 0; c < 3; ++c) {
    int M, N, K;
    dims_of(c, &M, &N, &K);
    for (int m = 0; m < M; ++m)
      for (int n = 0; n < N; ++n) {
        int s = 0;
        for (int k = 0; k < K; ++k) s += a_val(c, m, k) * b_val(c, k, n);
        out[off + m * N + n] = (float)s;
      }
    off += M * N;
  }
}

// Number of entries of `got` (same packing) that differ from the expected
// products; 0 when every layout is the assumed one.
inline int count_mismatches(const float* got) {
  float want[kOutFloats];
  expected(want);
  int bad = 0;
  for (int e = 0; e < kOutFloats; ++e) bad += got[e] != want[e];
  return bad;
}

}  // namespace selftest
}  // namespace dsa
