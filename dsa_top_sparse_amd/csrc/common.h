// common.h -- device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Order-preserving map of an fp32 score to uint32: a > b (as floats) iff
// key(a) > key(b). -0.0 is folded onto +0.0 first so that the two compare
// equal, as they do as floats.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Debug builds (-DDSA_LDS_POISON) fill the workgroup's LDS -- the static part
// and `dyn_bytes` of dynamic LDS after it -- with a NaN pattern before the
// kernel body runs, so that a read of LDS the kernel never wrote shows in its
// results. Every kernel calls it first, before any early return (it ends in a
// barrier); the product build compiles it to nothing.
__device__ __forceinline__ void lds_poison(uint32_t dyn_bytes = 0) {
#ifdef DSA_LDS_POISON
  const uint32_t words = (__builtin_amdgcn_groupstaticsize() + dyn_bytes) / 4u;
  for (uint32_t w = threadIdx.x; w < words; w += blockDim.x)
    asm volatile("ds_write_b32 %0, %1" ::"v"(4u * w), "v"(0x7FC00001u) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
#else
  (void)dyn_bytes;
#endif
}

}  // namespace dsa
