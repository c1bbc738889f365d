// validate.h -- host-side argument checks of every C ABI call. No HIP: this
// part builds for the host alone (the CPU tests also run it under ASan and
// UBSan). Each check returns DSA_OK and fills the step's arguments, or the
// status the call must return without touching the device.
#pragma once

#include "args.h"
#include "dsa.h"

namespace dsa {

dsa_status check_indexer(const dsa_dims* dims, const void* q_idx, const float* w_idx, const void* k_idx_cache,
                         float* scores, int64_t ld, IndexerArgs* a);
dsa_status check_topk(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, size_t ws_bytes,
                      TopkArgs* a);
dsa_status check_mla(const dsa_dims* dims, const void* q, const void* kv_cache, const int32_t* idx, float* out,
                     float* lse, MlaArgs* a);
// Extra checks of the cache append of a prefill chunk (after the three steps'
// checks): the chunk rows' pointers and their placement against the caches.
dsa_status check_append(const dsa_dims* dims, const void* kv_chunk, const void* k_idx_chunk, const void* kv_cache,
                        const void* k_idx_cache);
// Workspace of a decode call: DSA_OK when `ws_bytes` at `workspace` holds
// `need` bytes (need == 0 accepts anything).
dsa_status check_workspace(const void* workspace, size_t ws_bytes, size_t need);

// The fused indexer + select: the indexer's and the select's checks (no score
// matrix argument), the output and the workspace; fills both steps' arguments
// and the workspace layout.
dsa_status check_indexer_topk(const dsa_dims* dims, const void* q_idx, const float* w_idx, const void* k_idx_cache,
                              int32_t* idx, const void* workspace, size_t ws_bytes, IndexerArgs* ia, TopkArgs* ta,
                              FusedLayout* layout);

size_t act_row_bytes(const dsa_dims* dims);  // one latent cache row
size_t idx_row_bytes(const dsa_dims* dims);  // one indexer-key cache row

}  // namespace dsa
