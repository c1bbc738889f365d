// validate.cpp -- argument checks of the C ABI (include/dsa.h). Host-only
// C++: nothing here touches the device, so an invalid call is rejected before
// anything is enqueued.
#include "validate.h"

#include <math.h>

namespace dsa {

namespace {

constexpr int64_t kMaxPos = 0x7fffffffLL;  // positions and cache rows are int32

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == DSA_BF16 || d == DSA_F32; }

// Checks shared by every call: counts, positions.
dsa_status check_chunk(const dsa_dims* d) {
  if (!d) return DSA_ERR_NULL;
  if (d->n_q < 0 || d->offset < 0) return DSA_ERR_SHAPE;
  if ((int64_t)d->offset + d->n_q > kMaxPos) return DSA_ERR_SHAPE;
  return DSA_OK;
}

size_t dtype_bytes(int32_t d) { return d == DSA_BF16 ? 2 : 4; }

// [a, a + n) and [b, b + n) overlap without being the same range.
bool partial_overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x != y && x < y + n && y < x + n;
}

}  // namespace

bool indexer_fast_path(const IndexerArgs& a) {
  return a.bf16 && a.n_idx_heads == 4 && (a.d_idx == 32 || a.d_idx == 64 || a.d_idx == 128 || a.d_idx == 256);
}

bool mla_fast_path(const MlaArgs& a) {
  // top_k % 4 == 0: the index ring is filled with 16-byte loads from 16-byte
  // aligned rows. The cache must stay below 4 GiB (32-bit byte offsets).
  return a.bf16 && a.n_heads == 64 && a.d_latent == 512 && a.d_rope == 64 && a.top_k % 4 == 0 &&
         (int64_t)(a.offset + a.n_q) * 1152 < ((int64_t)1 << 32);
}

MlaSplit mla_decode_split(const MlaArgs& a) {
  MlaSplit sp{1, a.top_k};
  if (!mla_fast_path(a) || a.n_q <= 0) return sp;
  // enough workgroups to occupy the chip (one per CU), splits of whole tiles
  const int want = (kDecodeTargetGroups + a.n_q - 1) / a.n_q;
  const int max_splits = (a.top_k + kDecodeMinSlots - 1) / kDecodeMinSlots;
  const int splits = want < max_splits ? want : max_splits;
  if (splits <= 1) return sp;
  int slots = (a.top_k + splits - 1) / splits;
  slots = (slots + kDecodeTile - 1) / kDecodeTile * kDecodeTile;
  sp.splits = (a.top_k + slots - 1) / slots;
  sp.split_slots = slots;
  return sp;
}

size_t mla_decode_workspace_bytes(const MlaArgs& a) {
  const MlaSplit sp = mla_decode_split(a);
  if (sp.splits <= 1) return 0;
  return (size_t)sp.splits * (size_t)a.n_q * (size_t)a.n_heads * (size_t)(a.d_latent + 1) * sizeof(float);
}

IndexerUnits indexer_units(int n_q, int64_t ld) {
  const int n_qb = (n_q + 63) / 64;
  // Aim for >= 2048 workgroups (8 per CU) with 64-key-aligned ranges.
  const int64_t target_ranges = (2048 + n_qb - 1) / n_qb;
  int64_t kpu = (ld + target_ranges - 1) / target_ranges;
  kpu = ((kpu + 63) / 64) * 64;
  if (kpu < 128) kpu = 128;
  if (kpu > 1024) kpu = 1024;
  return IndexerUnits{n_qb, static_cast<int>(kpu), (ld + kpu - 1) / kpu};
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

FusedLayout fused_layout(int n_q, int offset, int n_idx_heads, int d_idx, bool idx_bf16, int top_k) {
  FusedLayout L{};
  const int64_t t_ctx = static_cast<int64_t>(offset) + n_q;
  const IndexerUnits un = indexer_units(n_q, t_ctx);
  const int64_t row_cap = un.n_kr * un.keys_per_unit;
  L.fused = idx_bf16 && n_idx_heads == 4 && d_idx == 128 && t_ctx <= kFusedMaxRow && top_k <= kFusedMaxTopk &&
            static_cast<int64_t>(n_q) * row_cap < (int64_t(1) << 32);
  if (L.fused) {
    size_t o = 0;
    L.tau_off = o;
    o = align256(o + 4 * static_cast<size_t>(n_q));
    L.tf_off = o;
    o = align256(o + 4 * static_cast<size_t>(n_q));
    L.counts_off = o;
    o = align256(o + 4 * static_cast<size_t>(n_q) * static_cast<size_t>(un.n_kr));
    L.sample_off = o;
    o = align256(o + 4 * static_cast<size_t>(n_q) * kFusedSample);
    L.cand_off = o;
    o = align256(o + 8 * static_cast<size_t>(n_q) * static_cast<size_t>(row_cap));
    L.bytes = o;
    L.row_cap = row_cap;
    L.n_kr = un.n_kr;
    L.keys_per_unit = un.keys_per_unit;
  } else {
    L.scores_ld = (t_ctx + 3) & ~int64_t(3);
    L.scores_off = 0;
    L.bytes = align256(4 * static_cast<size_t>(n_q) * static_cast<size_t>(L.scores_ld));
  }
  return L;
}

dsa_status check_indexer(const dsa_dims* dims, const void* q_idx, const float* w_idx, const void* k_idx_cache,
                         float* scores, int64_t ld, IndexerArgs* a) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->n_idx_heads <= 0 || dims->d_idx <= 0) return DSA_ERR_SHAPE;
  if (!valid_dtype(dims->idx_dtype)) return DSA_ERR_DTYPE;
  if (ld < (int64_t)dims->offset + dims->n_q) return DSA_ERR_SHAPE;
  if (dims->n_q == 0) return DSA_OK;
  if (!q_idx || !w_idx || !k_idx_cache || !scores) return DSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx_cache) || !aligned16(scores))
    return DSA_ERR_ALIGN;
  *a = IndexerArgs{dims->n_q, dims->offset, dims->n_idx_heads, dims->d_idx, dims->idx_dtype == DSA_BF16,
                   q_idx, w_idx, k_idx_cache, scores, ld};
  if (!indexer_fast_path(*a)) {
    if ((int64_t)dims->n_idx_heads * dims->d_idx > kPlainIndexerMaxElems) return DSA_ERR_UNSUPPORTED;
    if (dims->n_q > 65535 || (ld + 255) / 256 > kMaxPos) return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

dsa_status check_topk(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, size_t ws_bytes,
                      TopkArgs* a) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->top_k < 1 || dims->top_k > kTopkMax) return DSA_ERR_SHAPE;
  if (ld < (int64_t)dims->offset + dims->n_q) return DSA_ERR_SHAPE;
  (void)ws_bytes;  // the select needs no workspace
  if (dims->n_q == 0) return DSA_OK;
  if (!scores || !idx) return DSA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(idx)) return DSA_ERR_ALIGN;
  *a = TopkArgs{dims->n_q, dims->offset, dims->top_k, scores, ld, idx};
  return DSA_OK;
}

dsa_status check_mla(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx, float* out,
                     float* lse, MlaArgs* a) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->n_heads <= 0 || dims->d_latent <= 0 || dims->d_rope < 0 || dims->top_k < 1 || dims->top_k > kTopkMax)
    return DSA_ERR_SHAPE;
  if (!isfinite(dims->sm_scale)) return DSA_ERR_SHAPE;
  if (!valid_dtype(dims->act_dtype)) return DSA_ERR_DTYPE;
  if (dims->n_q == 0) return DSA_OK;
  if (!q || !kv_cache || !idx || !out) return DSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(idx) || !aligned16(out) || (lse && !aligned16(lse)))
    return DSA_ERR_ALIGN;
  *a = MlaArgs{dims->n_q, dims->offset, dims->n_heads, dims->d_latent, dims->d_rope, dims->top_k,
               dims->sm_scale, dims->act_dtype == DSA_BF16, q, kv_cache, idx, out, lse};
  if (!mla_fast_path(*a)) {
    if ((int64_t)dims->d_latent + dims->d_rope > kPlainMlaMaxDqk || dims->top_k > kPlainMlaMaxTopk ||
        dims->n_heads > 65535)
      return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

dsa_status check_indexer_topk(const dsa_dims* dims, const void* q_idx, const float* w_idx, const void* k_idx_cache,
                              int32_t* idx, const void* workspace, size_t ws_bytes, IndexerArgs* ia, TopkArgs* ta,
                              FusedLayout* layout) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  const int64_t t_ctx = static_cast<int64_t>(dims->offset) + dims->n_q;
  // the indexer's checks with the workspace standing in for the score matrix
  // (pointers checked below), then the select's
  st = check_indexer(dims, q_idx, w_idx, k_idx_cache, reinterpret_cast<float*>(16), t_ctx, ia);
  if (st != DSA_OK) return st;
  st = check_topk(dims, reinterpret_cast<const float*>(16), t_ctx, idx, 0, ta);
  if (st != DSA_OK) return st;
  if (dims->n_q == 0) return DSA_OK;
  *layout = fused_layout(dims->n_q, dims->offset, dims->n_idx_heads, dims->d_idx, dims->idx_dtype == DSA_BF16,
                         dims->top_k);
  return check_workspace(workspace, ws_bytes, layout->bytes);
}

size_t act_row_bytes(const dsa_dims* dims) { return dtype_bytes(dims->act_dtype) * (size_t)(dims->d_latent + dims->d_rope); }
size_t idx_row_bytes(const dsa_dims* dims) { return dtype_bytes(dims->idx_dtype) * (size_t)dims->d_idx; }

dsa_status check_append(const dsa_dims* dims, const void* kv_chunk, const void* k_idx_chunk, const void* kv_cache,
                        const void* k_idx_cache) {
  if (!kv_chunk || !k_idx_chunk || !kv_cache || !k_idx_cache) return DSA_ERR_NULL;
  if (!aligned16(kv_chunk) || !aligned16(k_idx_chunk) || !aligned16(k_idx_cache)) return DSA_ERR_ALIGN;
  const size_t kv_row = act_row_bytes(dims), kx_row = idx_row_bytes(dims);
  const uint8_t* kv_dst = static_cast<const uint8_t*>(kv_cache) + kv_row * (size_t)dims->offset;
  const uint8_t* kx_dst = static_cast<const uint8_t*>(k_idx_cache) + kx_row * (size_t)dims->offset;
  if (partial_overlap(kv_chunk, kv_dst, kv_row * (size_t)dims->n_q) ||
      partial_overlap(k_idx_chunk, kx_dst, kx_row * (size_t)dims->n_q))
    return DSA_ERR_SHAPE;
  return DSA_OK;
}

dsa_status check_workspace(const void* workspace, size_t ws_bytes, size_t need) {
  if (need == 0) return DSA_OK;
  if (!workspace || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

}  // namespace dsa
