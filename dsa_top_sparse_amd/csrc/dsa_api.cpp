// dsa_api.cpp -- the C ABI declared in include/dsa.h: argument validation,
// dispatch to the kernels, status reporting. Every check runs on the host
// before anything is enqueued, so an invalid call never touches the device.
#include "dsa.h"

#include <math.h>

#include "kernels.h"

namespace {

constexpr int64_t kMaxPos = 0x7fffffffLL;  // positions and cache rows are int32

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == DSA_BF16 || d == DSA_F32; }

// Checks shared by every call: counts, positions, dtypes of the chunk.
dsa_status check_chunk(const dsa_dims* d) {
  if (!d) return DSA_ERR_NULL;
  if (d->n_q < 0 || d->offset < 0) return DSA_ERR_SHAPE;
  if ((int64_t)d->offset + d->n_q > kMaxPos) return DSA_ERR_SHAPE;
  return DSA_OK;
}

dsa_status from_hip(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_DEVICE; }

}  // namespace

extern "C" {

dsa_status dsa_indexer_scores(const dsa_dims* dims, const void* q_idx, const float* w_idx,
                              const void* k_idx_cache, float* scores, int64_t ld, void* stream) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->n_idx_heads <= 0 || dims->d_idx <= 0) return DSA_ERR_SHAPE;
  if (!valid_dtype(dims->idx_dtype)) return DSA_ERR_DTYPE;
  if (ld < (int64_t)dims->offset + dims->n_q) return DSA_ERR_SHAPE;
  if (dims->n_q == 0) return DSA_OK;
  if (!q_idx || !w_idx || !k_idx_cache || !scores) return DSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx_cache) || !aligned16(scores))
    return DSA_ERR_ALIGN;
  dsa::IndexerArgs a{dims->n_q, dims->offset, dims->n_idx_heads, dims->d_idx, dims->idx_dtype == DSA_BF16,
                     q_idx, w_idx, k_idx_cache, scores, ld};
  if (!dsa::indexer_fast_path(a)) {
    if ((int64_t)dims->n_idx_heads * dims->d_idx > dsa::kPlainIndexerMaxElems) return DSA_ERR_UNSUPPORTED;
    if (dims->n_q > 65535 || (ld + 255) / 256 > kMaxPos) return DSA_ERR_UNSUPPORTED;
  }
  return from_hip(dsa::launch_indexer(a, static_cast<hipStream_t>(stream)));
}

size_t dsa_topk_workspace_bytes(const dsa_dims* dims) {
  (void)dims;
  return 0;  // the select keeps all of its state in LDS
}

dsa_status dsa_topk_select(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, void* workspace,
                           size_t ws_bytes, void* stream) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->top_k < 1 || dims->top_k > dsa::kTopkMax) return DSA_ERR_SHAPE;
  if (ld < (int64_t)dims->offset + dims->n_q) return DSA_ERR_SHAPE;
  if (ws_bytes < dsa_topk_workspace_bytes(dims)) return DSA_ERR_WORKSPACE;
  (void)workspace;
  if (dims->n_q == 0) return DSA_OK;
  if (!scores || !idx) return DSA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(idx)) return DSA_ERR_ALIGN;
  dsa::TopkArgs a{dims->n_q, dims->offset, dims->top_k, scores, ld, idx};
  return from_hip(dsa::launch_topk(a, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_sparse_mla_fwd(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx,
                              float* out, float* lse, void* stream) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->n_heads <= 0 || dims->d_latent <= 0 || dims->d_rope < 0 || dims->top_k < 1 ||
      dims->top_k > dsa::kTopkMax)
    return DSA_ERR_SHAPE;
  if (!isfinite(dims->sm_scale)) return DSA_ERR_SHAPE;
  if (!valid_dtype(dims->act_dtype)) return DSA_ERR_DTYPE;
  if (dims->n_q == 0) return DSA_OK;
  if (!q || !kv_cache || !idx || !out) return DSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(idx) || !aligned16(out) || (lse && !aligned16(lse)))
    return DSA_ERR_ALIGN;
  dsa::MlaArgs a{dims->n_q, dims->offset, dims->n_heads, dims->d_latent, dims->d_rope, dims->top_k,
                 dims->sm_scale, dims->act_dtype == DSA_BF16, q, kv_cache, idx, out, lse};
  if (!dsa::mla_fast_path(a)) {
    if ((int64_t)dims->d_latent + dims->d_rope > dsa::kPlainMlaMaxDqk || dims->top_k > dsa::kPlainMlaMaxTopk ||
        dims->n_heads > 65535)
      return DSA_ERR_UNSUPPORTED;
  }
  return from_hip(dsa::launch_mla(a, static_cast<hipStream_t>(stream)));
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "unknown dtype code";
    case DSA_ERR_UNSUPPORTED: return "shape not supported by any kernel of this library";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_DEVICE: return "HIP reported an error while launching";
    case DSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
  }
  return "unknown status";
}

int32_t dsa_version(void) { return 100; }

}  // extern "C"
