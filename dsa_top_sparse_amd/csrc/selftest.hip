// selftest.hip -- checks run once per device before the first fast-path
// launch:
//   * the matrix-core layout self-test: known products through the MFMA
//     forms and operand paths the kernels use (operands and expected values in
//     selftest_ref.h), so that a layout the kernels do not expect (for
//     example a transposed operand) is reported instead of producing wrong
//     scores or outputs;
//   * launch limits: each fast kernel's block size, LDS and registers against
//     what the device allows (the pages report a sparse-attention kernel
//     launched past a pipeline's thread limit: TensorFold issue #743, the
//     pre-M5 kernel checks).
#include <mutex>
#include <unordered_map>

#include "common.h"
#include "device_checks.h"
#include "kernels.h"
#include "selftest_ref.h"

namespace dsa {

namespace {

__device__ float g_selftest_out[selftest::kOutFloats];

__device__ __forceinline__ __bf16 bfi(int v) { return static_cast<__bf16>(static_cast<float>(v)); }

// One wave. Fragment layouts as the fast kernels assume them:
//   16x16x32: A lane l holds row l%16, k = 8 (l/16) + e; B lane l holds
//             column l%16, same k; C lane l holds column l%16, rows 4 (l/16) + r.
//   32x32x16: A lane l holds row l%32, k = 8 (l/32) + e; B column l%32, same k;
//             C lane l holds column l%32, rows 8 (r/4) + 4 (l/32) + r%4.
//   case 2:   B (32 x 16, row-major in LDS, 32 bytes a row) read with the
//             transposing LDS read the attention's P V uses: lane (4e + c) of
//             16-lane group G reads 4 values of row 8G + 4h + e at column 4c,
//             and receives column l%16 of rows 8G + 4h .. +3.
__global__ __launch_bounds__(64) void mfma_selftest_kernel() {
  __shared__ __attribute__((aligned(16))) uint16_t vt[32 * 16];
  const int l = threadIdx.x;
  // ---- case 0
  {
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
      a[e] = bfi(selftest::a_val(0, l % 16, 8 * (l / 16) + e));
      b[e] = bfi(selftest::b_val(0, 8 * (l / 16) + e, l % 16));
    }
    f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0, 0, 0, 0}, 0, 0, 0);
    for (int r = 0; r < 4; ++r) g_selftest_out[(4 * (l / 16) + r) * 16 + l % 16] = c[r];
  }
  // ---- case 1
  {
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
      a[e] = bfi(selftest::a_val(1, l % 32, 8 * (l / 32) + e));
      b[e] = bfi(selftest::b_val(1, 8 * (l / 32) + e, l % 32));
    }
    f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, f32x16{}, 0, 0, 0);
    for (int r = 0; r < 16; ++r)
      g_selftest_out[selftest::kCase0 + (8 * (r / 4) + 4 * (l / 32) + r % 4) * 32 + l % 32] = c[r];
  }
  // ---- case 2
  {
    for (int e = l; e < 32 * 16; e += 64) {
      const float f = static_cast<float>(selftest::b_val(2, e / 16, e % 16));
      vt[e] = static_cast<uint16_t>(__float_as_uint(f) >> 16);  // small integers: exact in bf16
    }
    __syncthreads();
    bf16x8 a;
    for (int e = 0; e < 8; ++e) a[e] = bfi(selftest::a_val(2, l % 16, 8 * (l / 16) + e));
    const int l16 = l % 16, G = l / 16, e = l16 >> 2, c = l16 & 3;
    s16x4 d[2];
    for (int h = 0; h < 2; ++h) {
      const int byte = (8 * G + 4 * h + e) * 32 + 8 * c;
      d[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) uint8_t*)(
              (uintptr_t)(const __attribute__((address_space(3))) void*)vt) + byte));
    }
    const bf16x8 b = __builtin_bit_cast(bf16x8, (s16x8{d[0][0], d[0][1], d[0][2], d[0][3], d[1][0], d[1][1], d[1][2],
                                                       d[1][3]}));
    f32x4 o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, f32x4{0, 0, 0, 0}, 0, 0, 0);
    for (int r = 0; r < 4; ++r) g_selftest_out[selftest::kCase0 + selftest::kCase1 + (4 * G + r) * 16 + l16] = o[r];
  }
}

hipError_t run_self_test() {
  hipError_t e = launch_kernel(mfma_selftest_kernel, dim3(1), dim3(64), 0, nullptr);
  if (e != hipSuccess) return e;
  float got[selftest::kOutFloats];
  e = hipMemcpyFromSymbol(got, HIP_SYMBOL(g_selftest_out), sizeof got, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  return selftest::count_mismatches(got) == 0 ? hipSuccess : hipErrorInvalidValue;
}

}  // namespace

hipError_t once_per_device(PerDeviceCache& cache, hipError_t (*fn)()) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(cache.mu);
  auto it = cache.done.find(dev);
  if (it != cache.done.end()) return it->second;
  e = fn();
  cache.done.emplace(dev, e);
  return e;
}

hipError_t check_launch_limits(const void* kernel, int threads, size_t dyn_lds) {
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, kernel);
  if (e != hipSuccess) return e;
  int dev = 0, lds_max = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  if (attr.maxThreadsPerBlock < threads) return hipErrorInvalidConfiguration;
  if (attr.sharedSizeBytes + dyn_lds > (size_t)lds_max) return hipErrorInvalidConfiguration;
  if (attr.numRegs > 512) return hipErrorInvalidConfiguration;
  return hipSuccess;
}

hipError_t mfma_self_test() {
  static PerDeviceCache cache;
  return once_per_device(cache, run_self_test);
}

}  // namespace dsa
