// args.h -- validated arguments of each step, passed from the C ABI layer to
// the launchers. Plain C++ with no HIP types, so that the validation in
// validate.cpp builds and runs on the host alone (also under sanitizers).
#pragma once

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

// True when the MFMA indexer kernel handles these dims (bf16, 4 heads, width
// 32 / 64 / 128 / 256).
bool indexer_fast_path(const IndexerArgs& a);
// True when the MFMA attention kernel handles these dims (bf16, 64 heads,
// 512 + 64 dims, top_k % 4 == 0, cache below 4 GiB).
bool mla_fast_path(const MlaArgs& a);

// Largest d_idx * n_idx_heads / d_qk / top_k the plain kernels accept
// (their per-query rows live in LDS).
constexpr int kPlainIndexerMaxElems = 8192;
constexpr int kPlainMlaMaxDqk = 2048;
constexpr int kPlainMlaMaxTopk = 4096;
constexpr int kTopkMax = 1 << 20;

// Decode-shaped attention (few queries): each query's slots are split over
// several workgroups whose partial results a combine kernel merges.
struct MlaSplit {
  int splits;       // 1 = no split (plain launch)
  int split_slots;  // slots per split, a multiple of 32
};
constexpr int kDecodeTargetGroups = 256;  // workgroups to aim for
constexpr int kDecodeMinSlots = 128;      // smallest split
constexpr int kDecodeTile = 32;           // slots per tile of the attention kernel
MlaSplit mla_decode_split(const MlaArgs& a);
// Bytes of the partial outputs and log-sum-exps of a split launch (0 = no split).
size_t mla_decode_workspace_bytes(const MlaArgs& a);
// How the MFMA indexer splits a chunk of n_q queries over ld keys: 64-query
// blocks times ranges of keys_per_unit keys (n_kr of them).
struct IndexerUnits {
  int n_qb;
  int keys_per_unit;
  int64_t n_kr;
};
IndexerUnits indexer_units(int n_q, int64_t ld);

// Workspace of the fused indexer + select (dsa_indexer_topk). With `fused`
// (bf16 4 x 128 indexer, at most kFusedMaxRow keys, top_k <= kFusedMaxTopk),
// the byte offsets of its arrays; otherwise one [n_q][scores_ld] score matrix
// for the unfused kernels. Every array starts 256-byte aligned.
constexpr int kFusedMaxRow = 65536;  // candidate key indices are 16-bit in LDS
constexpr int kFusedMaxTopk = 4096;  // the select's LDS candidate capacity
constexpr int kFusedSample = 2048;   // keys of each query's threshold sample
struct FusedLayout {
  bool fused;
  size_t bytes;
  size_t tau_off, tf_off, counts_off, sample_off, cand_off;
  int64_t row_cap, n_kr;
  int keys_per_unit;
  size_t scores_off;
  int64_t scores_ld;
};
FusedLayout fused_layout(int n_q, int offset, int n_idx_heads, int d_idx, bool idx_bf16, int top_k);

// Size of the library's own decode scratch, used by the entry point that
// allocates nothing: 32 MiB holds 255 split partials of 64 heads x 513 fp32
// (e.g. up to 15 queries at 16 splits).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

}  // namespace dsa
