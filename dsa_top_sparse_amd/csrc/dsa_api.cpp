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

// Argument checks of each step, separated from the launch so that a call
// running several steps validates all of them before enqueuing anything.
dsa_status check_indexer(const dsa_dims* dims, const void* q_idx, const float* w_idx, const void* k_idx_cache,
                         float* scores, int64_t ld, dsa::IndexerArgs* a) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->n_idx_heads <= 0 || dims->d_idx <= 0) return DSA_ERR_SHAPE;
  if (!valid_dtype(dims->idx_dtype)) return DSA_ERR_DTYPE;
  if (ld < (int64_t)dims->offset + dims->n_q) return DSA_ERR_SHAPE;
  if (dims->n_q == 0) return DSA_OK;
  if (!q_idx || !w_idx || !k_idx_cache || !scores) return DSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx_cache) || !aligned16(scores))
    return DSA_ERR_ALIGN;
  *a = dsa::IndexerArgs{dims->n_q, dims->offset, dims->n_idx_heads, dims->d_idx, dims->idx_dtype == DSA_BF16,
                        q_idx, w_idx, k_idx_cache, scores, ld};
  if (!dsa::indexer_fast_path(*a)) {
    if ((int64_t)dims->n_idx_heads * dims->d_idx > dsa::kPlainIndexerMaxElems) return DSA_ERR_UNSUPPORTED;
    if (dims->n_q > 65535 || (ld + 255) / 256 > kMaxPos) return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

dsa_status check_topk(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, size_t ws_bytes,
                      dsa::TopkArgs* a) {
  dsa_status st = check_chunk(dims);
  if (st != DSA_OK) return st;
  if (dims->top_k < 1 || dims->top_k > dsa::kTopkMax) return DSA_ERR_SHAPE;
  if (ld < (int64_t)dims->offset + dims->n_q) return DSA_ERR_SHAPE;
  if (ws_bytes < dsa_topk_workspace_bytes(dims)) return DSA_ERR_WORKSPACE;
  if (dims->n_q == 0) return DSA_OK;
  if (!scores || !idx) return DSA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(idx)) return DSA_ERR_ALIGN;
  *a = dsa::TopkArgs{dims->n_q, dims->offset, dims->top_k, scores, ld, idx};
  return DSA_OK;
}

dsa_status check_mla(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx, float* out,
                     float* lse, dsa::MlaArgs* a) {
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
  *a = dsa::MlaArgs{dims->n_q, dims->offset, dims->n_heads, dims->d_latent, dims->d_rope, dims->top_k,
                    dims->sm_scale, dims->act_dtype == DSA_BF16, q, kv_cache, idx, out, lse};
  if (!dsa::mla_fast_path(*a)) {
    if ((int64_t)dims->d_latent + dims->d_rope > dsa::kPlainMlaMaxDqk || dims->top_k > dsa::kPlainMlaMaxTopk ||
        dims->n_heads > 65535)
      return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

size_t dtype_bytes(int32_t d) { return d == DSA_BF16 ? 2 : 4; }

// [src, src + n) and [dst, dst + n) overlap without being the same range.
bool partial_overlap(const void* src, const void* dst, size_t n) {
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  return s != d && s < d + n && d < s + n;
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_scores(const dsa_dims* dims, const void* q_idx, const float* w_idx,
                              const void* k_idx_cache, float* scores, int64_t ld, void* stream) {
  dsa::IndexerArgs a{};
  const dsa_status st = check_indexer(dims, q_idx, w_idx, k_idx_cache, scores, ld, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  return from_hip(dsa::launch_indexer(a, static_cast<hipStream_t>(stream)));
}

size_t dsa_topk_workspace_bytes(const dsa_dims* dims) {
  (void)dims;
  return 0;  // the select keeps all of its state in LDS
}

dsa_status dsa_topk_select(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, void* workspace,
                           size_t ws_bytes, void* stream) {
  (void)workspace;
  dsa::TopkArgs a{};
  const dsa_status st = check_topk(dims, scores, ld, idx, ws_bytes, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  return from_hip(dsa::launch_topk(a, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_sparse_mla_fwd(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx,
                              float* out, float* lse, void* stream) {
  dsa::MlaArgs a{};
  const dsa_status st = check_mla(dims, q, kv_cache, idx, out, lse, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  return from_hip(dsa::launch_mla(a, static_cast<hipStream_t>(stream)));
}

size_t dsa_sparse_mla_decode_workspace_bytes(const dsa_dims* dims) {
  if (check_chunk(dims) != DSA_OK || dims->n_q <= 0 || dims->top_k < 1 || dims->top_k > dsa::kTopkMax) return 0;
  dsa::MlaArgs a{dims->n_q, dims->offset, dims->n_heads, dims->d_latent, dims->d_rope, dims->top_k,
                 dims->sm_scale, dims->act_dtype == DSA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr};
  return dsa::mla_decode_workspace_bytes(a);
}

dsa_status dsa_sparse_mla_decode(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx,
                                 float* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  dsa::MlaArgs a{};
  const dsa_status st = check_mla(dims, q, kv_cache, idx, out, lse, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  const size_t need = dsa::mla_decode_workspace_bytes(a);
  if (need > 0) {
    if (!workspace || ws_bytes < need) return DSA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  }
  return from_hip(dsa::launch_mla_decode(a, workspace, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_prefill_chunk(const dsa_dims* dims, const void* q, const void* kv_chunk, const void* q_idx,
                             const float* w_idx, const void* k_idx_chunk, void* kv_cache, void* k_idx_cache,
                             float* scores, int64_t ld, int32_t* idx, float* out, float* lse, void* workspace,
                             size_t ws_bytes, void* stream) {
  dsa::IndexerArgs ia{};
  dsa::TopkArgs ta{};
  dsa::MlaArgs ma{};
  dsa_status st = check_indexer(dims, q_idx, w_idx, k_idx_cache, scores, ld, &ia);
  if (st == DSA_OK) st = check_topk(dims, scores, ld, idx, ws_bytes, &ta);
  if (st == DSA_OK) st = check_mla(dims, q, kv_cache, idx, out, lse, &ma);
  if (st != DSA_OK || dims->n_q == 0) return st;
  (void)workspace;
  if (!kv_chunk || !k_idx_chunk) return DSA_ERR_NULL;
  if (!aligned16(kv_chunk) || !aligned16(k_idx_chunk)) return DSA_ERR_ALIGN;
  const size_t kv_row = dtype_bytes(dims->act_dtype) * (size_t)(dims->d_latent + dims->d_rope);
  const size_t kx_row = dtype_bytes(dims->idx_dtype) * (size_t)dims->d_idx;
  uint8_t* kv_dst = static_cast<uint8_t*>(kv_cache) + kv_row * (size_t)dims->offset;
  uint8_t* kx_dst = static_cast<uint8_t*>(k_idx_cache) + kx_row * (size_t)dims->offset;
  const size_t kv_bytes = kv_row * (size_t)dims->n_q, kx_bytes = kx_row * (size_t)dims->n_q;
  if (partial_overlap(kv_chunk, kv_dst, kv_bytes) || partial_overlap(k_idx_chunk, kx_dst, kx_bytes))
    return DSA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // append the chunk's rows (skipped when the caller wrote them in place)
  if (kv_chunk != kv_dst && hipMemcpyAsync(kv_dst, kv_chunk, kv_bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return DSA_ERR_DEVICE;
  if (k_idx_chunk != kx_dst &&
      hipMemcpyAsync(kx_dst, k_idx_chunk, kx_bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return DSA_ERR_DEVICE;
  if (dsa::launch_indexer(ia, s) != hipSuccess) return DSA_ERR_DEVICE;
  if (dsa::launch_topk(ta, s) != hipSuccess) return DSA_ERR_DEVICE;
  return from_hip(dsa::launch_mla(ma, s));
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
