// kernels.h -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct IndexerArgs {
  int n_q, offset, n_idx_heads, d_idx;
  bool bf16;
  const void* q_idx;
  const float* w;
  const void* k_idx;
  float* scores;
  int64_t ld;
};

struct TopkArgs {
  int n_q, offset, top_k;
  const float* scores;
  int64_t ld;
  int32_t* idx;
};

struct MlaArgs {
  int n_q, offset, n_heads, d_latent, d_rope, top_k;
  float sm_scale;
  bool bf16;
  const void* q;
  const void* kv;
  const int32_t* idx;
  float* out;
  float* lse;
};

// True when the MFMA indexer kernel handles these dims.
bool indexer_fast_path(const IndexerArgs& a);
// True when the MFMA attention kernel handles these dims.
bool mla_fast_path(const MlaArgs& a);
// Largest d_idx * n_idx_heads / d_qk the plain kernels accept (LDS-resident rows).
constexpr int kPlainIndexerMaxElems = 8192;
constexpr int kPlainMlaMaxDqk = 2048;
constexpr int kPlainMlaMaxTopk = 4096;
constexpr int kTopkMax = 1 << 20;

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_mla(const MlaArgs& a, hipStream_t s);

// Decode-shaped attention (few queries): each query's slots are split over
// several workgroups whose partial results a combine kernel merges.
struct MlaSplit {
  int splits;       // 1 = no split (plain launch)
  int split_slots;  // slots per split, a multiple of 32
};
constexpr int kDecodeTargetGroups = 256;  // workgroups to aim for
constexpr int kDecodeMinSlots = 128;      // smallest split
MlaSplit mla_decode_split(const MlaArgs& a);
size_t mla_decode_workspace_bytes(const MlaArgs& a);
hipError_t launch_mla_decode(const MlaArgs& a, void* workspace, hipStream_t s);

}  // namespace dsa
