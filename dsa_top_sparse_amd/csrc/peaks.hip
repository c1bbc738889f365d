// peaks.hip -- measurement micro-kernels, not part of the DSA path: the dense
// bf16 matrix-core rate and the HBM copy rate this device reaches, measured
// beside the published peaks (the feedman.me page measures its machines' raw
// matmul and streaming rates the same way). Built into a library of its own,
// libdsa_peaks.so, that only the benchmark loads.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 1024;  // 16 waves: four per SIMD
constexpr int kChains = 8;          // independent accumulators per wave

// Each wave runs iters x 16 x kChains 16x16x32 bf16 products (16,384 flop
// each) on register operands; the sums go to `sink` so that nothing is
// removed.
__global__ __launch_bounds__(kMfmaThreads) void peak_mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>((threadIdx.x + i) & 7) * 0.125f);
    b[i] = static_cast<__bf16>(static_cast<float>(i) - 3.5f);
  }
  f32x4 acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, static_cast<float>(c)};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[static_cast<size_t>(blockIdx.x) * kMfmaThreads + threadIdx.x] = s;
}

constexpr int kCopyThreads = 256;

// dst = src, 16 bytes per lane per step, grid-stride; n16 = bytes / 16.
__global__ __launch_bounds__(kCopyThreads) void peak_copy_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kCopyThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kCopyThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Enqueues the matrix-core loop on `stream` (a hipStream_t): `blocks`
// workgroups of 16 waves; `sink` holds blocks * 1024 floats. Flop per launch:
// blocks * 16 * iters * 16 * 8 * 16,384. Returns the launch's hipError_t.
__attribute__((visibility("default"))) int dsa_peak_mfma(int blocks, int iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !sink) return static_cast<int>(hipErrorInvalidValue);
  void* args[] = {&iters, &sink};
  return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void*>(peak_mfma_kernel), dim3(blocks),
                                          dim3(kMfmaThreads), args, 0, static_cast<hipStream_t>(stream)));
}

// Enqueues dst = src for `bytes` (a multiple of 16; both pointers 16-byte
// aligned device memory) on `stream`. Returns the launch's hipError_t.
__attribute__((visibility("default"))) int dsa_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return static_cast<int>(hipErrorInvalidValue);
  size_t n16 = bytes / 16;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  void* args[] = {&s, &d, &n16};
  return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void*>(peak_copy_kernel), dim3(256 * 16),
                                          dim3(kCopyThreads), args, 0, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
