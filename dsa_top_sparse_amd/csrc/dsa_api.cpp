// dsa_api.cpp -- the C ABI declared in include/dsa.h: dispatch to the kernels
// after the host-side argument checks of validate.cpp, status reporting, and
// the once-per-device checks (matrix-core layout self-test, launch limits).
#include "dsa.h"

#include "kernels.h"
#include "validate.h"

namespace {

dsa_status from_hip(hipError_t e) {
  if (e == hipSuccess) return DSA_OK;
  return e == hipErrorInvalidConfiguration ? DSA_ERR_UNSUPPORTED : DSA_ERR_DEVICE;
}

enum Step { kIndexer = 1, kTopk = 2, kMla = 4, kFused = 8 };

// The checks that must pass before the first launch of the given steps on
// this device: the launch limits of their kernels and, unless the stream is
// being captured into a graph (the self-test synchronises), the matrix-core
// layout self-test. Each runs once per device; later calls only read the
// cached results.
dsa_status ready(int steps, hipStream_t s) {
  hipError_t e = hipSuccess;
  if ((steps & kIndexer) && e == hipSuccess) e = dsa::check_indexer_kernels();
  if ((steps & kTopk) && e == hipSuccess) e = dsa::check_topk_kernels();
  if ((steps & kMla) && e == hipSuccess) e = dsa::check_mla_kernels();
  if ((steps & kFused) && e == hipSuccess) e = dsa::check_fused_kernels();
  if (e != hipSuccess) return from_hip(e);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return DSA_ERR_DEVICE;
  if (cap == hipStreamCaptureStatusNone) return from_hip(dsa::mfma_self_test());
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_indexer_scores(const dsa_dims* dims, const void* q_idx, const float* w_idx,
                              const void* k_idx_cache, float* scores, int64_t ld, void* stream) {
  dsa::IndexerArgs a{};
  dsa_status st = dsa::check_indexer(dims, q_idx, w_idx, k_idx_cache, scores, ld, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kIndexer, s)) != DSA_OK) return st;
  return from_hip(dsa::launch_indexer(a, s));
}

size_t dsa_topk_workspace_bytes(const dsa_dims* dims) {
  (void)dims;
  return 0;  // the select keeps all of its state in LDS
}

dsa_status dsa_topk_select(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, void* workspace,
                           size_t ws_bytes, void* stream) {
  (void)workspace;
  dsa::TopkArgs a{};
  dsa_status st = dsa::check_topk(dims, scores, ld, idx, ws_bytes, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kTopk, s)) != DSA_OK) return st;
  return from_hip(dsa::launch_topk(a, s));
}

size_t dsa_indexer_topk_workspace_bytes(const dsa_dims* dims) {
  if (!dims || dims->n_q <= 0 || dims->offset < 0 || (int64_t)dims->offset + dims->n_q > 0x7fffffffLL ||
      dims->top_k < 1 || dims->top_k > dsa::kTopkMax || dims->n_idx_heads <= 0 || dims->d_idx <= 0)
    return 0;
  return dsa::fused_layout(dims->n_q, dims->offset, dims->n_idx_heads, dims->d_idx, dims->idx_dtype == DSA_BF16,
                           dims->top_k)
      .bytes;
}

dsa_status dsa_indexer_topk(const dsa_dims* dims, const void* q_idx, const float* w_idx, const void* k_idx_cache,
                            int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
  dsa::IndexerArgs ia{};
  dsa::TopkArgs ta{};
  dsa::FusedLayout L{};
  dsa_status st = dsa::check_indexer_topk(dims, q_idx, w_idx, k_idx_cache, idx, workspace, ws_bytes, &ia, &ta, &L);
  if (st != DSA_OK || dims->n_q == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kIndexer | kTopk | (L.fused ? kFused : 0), s)) != DSA_OK) return st;
  return from_hip(dsa::launch_indexer_topk(ia, ta, L, workspace, s));
}

dsa_status dsa_sparse_mla_fwd(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx,
                              float* out, float* lse, void* stream) {
  dsa::MlaArgs a{};
  dsa_status st = dsa::check_mla(dims, q, kv_cache, idx, out, lse, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kMla, s)) != DSA_OK) return st;
  return from_hip(dsa::launch_mla(a, s));
}

size_t dsa_sparse_mla_decode_workspace_bytes(const dsa_dims* dims) {
  if (!dims || dims->n_q <= 0 || dims->offset < 0 || (int64_t)dims->offset + dims->n_q > 0x7fffffffLL ||
      dims->top_k < 1 || dims->top_k > dsa::kTopkMax)
    return 0;
  dsa::MlaArgs a{dims->n_q, dims->offset, dims->n_heads, dims->d_latent, dims->d_rope, dims->top_k,
                 dims->sm_scale, dims->act_dtype == DSA_BF16, nullptr, nullptr, nullptr, nullptr, nullptr};
  return dsa::mla_decode_workspace_bytes(a);
}

dsa_status dsa_sparse_mla_decode(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx,
                                 float* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  dsa::MlaArgs a{};
  dsa_status st = dsa::check_mla(dims, q, kv_cache, idx, out, lse, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  if ((st = dsa::check_workspace(workspace, ws_bytes, dsa::mla_decode_workspace_bytes(a))) != DSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kMla, s)) != DSA_OK) return st;
  return from_hip(dsa::launch_mla_decode(a, workspace, s));
}

dsa_status dsa_sparse_mla_decode_noalloc(const dsa_dims* dims, const void* q, const void* kv_cache,
                                         const int32_t* idx, float* out, float* lse, void* stream) {
  dsa::MlaArgs a{};
  dsa_status st = dsa::check_mla(dims, q, kv_cache, idx, out, lse, &a);
  if (st != DSA_OK || dims->n_q == 0) return st;
  const size_t need = dsa::mla_decode_workspace_bytes(a);
  if (need > dsa::kDecodeScratchBytes) return DSA_ERR_WORKSPACE;  // beyond the library's scratch
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kMla, s)) != DSA_OK) return st;
  void* ws = nullptr;
  if (need > 0 && dsa::decode_scratch(&ws) != hipSuccess) return DSA_ERR_DEVICE;
  return from_hip(dsa::launch_mla_decode(a, ws, s));
}

dsa_status dsa_prefill_chunk(const dsa_dims* dims, const void* q, const void* kv_chunk, const void* q_idx,
                             const float* w_idx, const void* k_idx_chunk, void* kv_cache, void* k_idx_cache,
                             float* scores, int64_t ld, int32_t* idx, float* out, float* lse, void* workspace,
                             size_t ws_bytes, void* stream) {
  dsa::IndexerArgs ia{};
  dsa::TopkArgs ta{};
  dsa::MlaArgs ma{};
  dsa::FusedLayout L{};
  const bool fused = scores == nullptr;  // steps 1-2 as dsa_indexer_topk
  dsa_status st = fused ? dsa::check_indexer_topk(dims, q_idx, w_idx, k_idx_cache, idx, workspace, ws_bytes, &ia,
                                                   &ta, &L)
                        : dsa::check_indexer(dims, q_idx, w_idx, k_idx_cache, scores, ld, &ia);
  if (st == DSA_OK && !fused) st = dsa::check_topk(dims, scores, ld, idx, ws_bytes, &ta);
  if (st == DSA_OK) st = dsa::check_mla(dims, q, kv_cache, idx, out, lse, &ma);
  if (st != DSA_OK || dims->n_q == 0) return st;
  if ((st = dsa::check_append(dims, kv_chunk, k_idx_chunk, kv_cache, k_idx_cache)) != DSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ready(kIndexer | kTopk | kMla | (fused && L.fused ? kFused : 0), s)) != DSA_OK) return st;
  const size_t kv_row = dsa::act_row_bytes(dims), kx_row = dsa::idx_row_bytes(dims);
  uint8_t* kv_dst = static_cast<uint8_t*>(kv_cache) + kv_row * (size_t)dims->offset;
  uint8_t* kx_dst = static_cast<uint8_t*>(k_idx_cache) + kx_row * (size_t)dims->offset;
  // append the chunk's rows (skipped when the caller wrote them in place)
  if (kv_chunk != kv_dst &&
      hipMemcpyAsync(kv_dst, kv_chunk, kv_row * (size_t)dims->n_q, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return DSA_ERR_DEVICE;
  if (k_idx_chunk != kx_dst &&
      hipMemcpyAsync(kx_dst, k_idx_chunk, kx_row * (size_t)dims->n_q, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return DSA_ERR_DEVICE;
  if (fused) {
    if ((st = from_hip(dsa::launch_indexer_topk(ia, ta, L, workspace, s))) != DSA_OK) return st;
  } else {
    if ((st = from_hip(dsa::launch_indexer(ia, s))) != DSA_OK) return st;
    if ((st = from_hip(dsa::launch_topk(ta, s))) != DSA_OK) return st;
  }
  return from_hip(dsa::launch_mla(ma, s));
}

dsa_status dsa_self_test(void) {
  const hipError_t e = dsa::mfma_self_test();
  if (e == hipSuccess) return DSA_OK;
  return DSA_ERR_DEVICE;
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "unknown dtype code";
    case DSA_ERR_UNSUPPORTED: return "shape not supported by any kernel of this library";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_DEVICE: return "HIP reported an error, or the device failed the matrix-core self-test";
    case DSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
  }
  return "unknown status";
}

int32_t dsa_version(void) { return 200; }

}  // extern "C"
