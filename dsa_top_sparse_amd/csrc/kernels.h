// kernels.h -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "args.h"

namespace dsa {

// Launches a kernel and returns the status of that launch itself (not an
// error left behind by an earlier, unrelated HIP call). The arguments are
// converted to the kernel's parameter types before their addresses are taken.
template <class T>
struct same_type {
  using type = T;
};
template <typename... KA>
hipError_t launch_kernel(void (*kernel)(KA...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                         typename same_type<KA>::type... args) {
  void* params[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, shmem, s);
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s);

// Output of the indexer's candidate mode (bf16, 4 x 128 only): for query i,
// the causal scores >= tf[i] of key range r, in key order, as (score bits,
// key index) pairs at cand[i * row_cap + r * keys_per_unit + 0 ..], their
// number at counts[i * n_kr + r]. Queries with offset + i + 1 <= top_k write
// nothing.
struct IndexerCandidates {
  const float* tf;
  uint2* cand;
  int32_t* counts;
  int64_t row_cap;  // n_kr * keys_per_unit
  int64_t n_kr;
  int top_k;
};
hipError_t launch_indexer_candidates(const IndexerArgs& a, const IndexerCandidates& fo, hipStream_t s);

// The fused indexer + select into idx (ta.idx) with the workspace laid out as
// L (ia.scores / ta.scores are ignored).
hipError_t launch_indexer_topk(const IndexerArgs& ia, const TopkArgs& ta, const FusedLayout& L, void* workspace,
                               hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_mla(const MlaArgs& a, hipStream_t s);
hipError_t launch_mla_decode(const MlaArgs& a, void* workspace, hipStream_t s);
// Device address of the current device's copy of the library's decode
// scratch (kDecodeScratchBytes), looked up once per device.
hipError_t decode_scratch(void** ptr);

// Launch-limit check of every fast-path kernel of a step on the current
// device (block size, LDS, registers against what the launch needs), cached
// per device after the first call. DSA_ERR_UNSUPPORTED-worthy failures return
// hipErrorInvalidConfiguration.
hipError_t check_indexer_kernels();
hipError_t check_topk_kernels();
hipError_t check_mla_kernels();
hipError_t check_fused_kernels();

// Runs the matrix-core layout self-test on the current device (once per
// device; later calls return the cached result). hipErrorInvalidValue when a
// product came out wrong.
hipError_t mfma_self_test();

}  // namespace dsa
