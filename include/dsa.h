/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA prefill hot path.
 *
 * One prompt chunk of n_q query tokens, appended at absolute position `offset`
 * to a per-token latent KV cache, goes through three calls:
 *
 *   dsa_indexer_scores  -> scores[n_q][ld]   (ReLU-weighted indexer score of every causal key)
 *   dsa_topk_select     -> idx[n_q][top_k]   (the top_k highest-scoring causal keys per query)
 *   dsa_sparse_mla_fwd  -> out[n_q][H][d_latent], lse[n_q][H]
 *                                            (softmax attention over only the selected rows)
 *
 * Source of the operation: the feedman.me page "GLM-5.3-Flash prefill on M5
 * Ultra, decode on M3 Ultra": its per-component profile (section "Per-component,
 * 8,192 tokens in 2,048-token chunks") names a "DSA indexer" and a "DSA
 * sparse-attention core"; the paragraph on what is not a matmul names the
 * per-query top-2,048 gather; the paragraph on the sparse-attention kernel
 * describes one query gathering its 2,048 keys; the hand-off paragraph gives
 * each token a latent KV row of 512 values. The pages print no formula, so the exact
 * definitions below are this library's contract (the same definitions as the
 * CPU oracle it is tested against).
 *
 * Query i (0 <= i < n_q) sits at absolute position p_i = offset + i. Its causal
 * keys are j = 0 .. p_i (a query sees itself). The caches hold
 * t_ctx = offset + n_q rows; the chunk's own rows are already written at
 * [offset, t_ctx).
 *
 * Conventions common to every call
 *  - Every pointer except `stream` is a DEVICE pointer owned by the caller. The
 *    library allocates nothing and keeps no per-call state.
 *  - Arrays are row-major and dense, with the shapes written beside each
 *    argument; base pointers must be 16-byte aligned.
 *  - bf16 arrays hold raw bfloat16 bit patterns (uint16_t).
 *  - `stream` is a hipStream_t (NULL = the default stream). All work is
 *    enqueued asynchronously on it; a call returns before the GPU finishes.
 *  - Errors: invalid arguments return a negative status BEFORE anything is
 *    enqueued; a failed launch returns DSA_ERR_DEVICE. Nothing aborts.
 *  - Before the first launch on a device each call checks its kernels'
 *    launch limits (block size, LDS, registers) against the device
 *    (DSA_ERR_UNSUPPORTED if one does not fit) and runs dsa_self_test.
 *  - Inputs are only read and outputs are only written; outputs must not alias
 *    inputs.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define DSA_API __attribute__((visibility("default")))
#else
#define DSA_API
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  DSA_ERR_DTYPE = -3,       /* unknown dtype code */
  DSA_ERR_UNSUPPORTED = -4, /* valid, but a shape no kernel here handles */
  DSA_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  DSA_ERR_DEVICE = -6,      /* HIP reported an error on launch */
  DSA_ERR_ALIGN = -7        /* a pointer is not 16-byte aligned */
} dsa_status;

typedef enum { DSA_BF16 = 0, DSA_F32 = 1 } dsa_dtype;

/* Shape of one chunk call. */
typedef struct {
  int32_t n_q;         /* queries in the chunk, >= 0 (0 = nothing to do) */
  int32_t offset;      /* absolute position of query 0, >= 0 */
  int32_t n_heads;     /* attention heads sharing one latent row per token */
  int32_t d_latent;    /* value width = the first d_latent dims of a latent row */
  int32_t d_rope;      /* key-only dims appended to each latent row (already rotated) */
  int32_t n_idx_heads; /* indexer heads */
  int32_t d_idx;       /* indexer head width; one shared indexer key row per token */
  int32_t top_k;       /* keys kept per query */
  float sm_scale;      /* softmax scale applied to q.k over all d_latent + d_rope dims */
  int32_t act_dtype;   /* dsa_dtype of q and the latent cache */
  int32_t idx_dtype;   /* dsa_dtype of the indexer queries and keys */
} dsa_dims;

/*
 * dsa_indexer_scores -- step 1, the DSA indexer.
 *
 *   scores[i][j] = sum_h w_idx[i][h] * max(0, sum_d q_idx[i][h][d] * k_idx[j][d])   j <= p_i
 *   scores[i][j] = -inf                                                             p_i < j < ld
 *
 * Arguments
 *   q_idx        [n_q][n_idx_heads][d_idx]   idx_dtype
 *   w_idx        [n_q][n_idx_heads]          fp32 (per query and indexer head)
 *   k_idx_cache  [offset + n_q][d_idx]       idx_dtype
 *   scores       [n_q][ld] fp32, written in full; ld >= offset + n_q
 * Products are accumulated in fp32. The result is exactly the real-number
 * value (bit-exact, +0.0 for zero) whenever every partial sum is an integer
 * of magnitude below 2^24, as with small-integer indexer inputs; otherwise it
 * is the fp32-rounded sum in an unspecified order.
 * Fast path: bf16 with n_idx_heads == 4 and d_idx a multiple of 32 (<= 256);
 * every other shape runs a plain kernel.
 */
DSA_API dsa_status dsa_indexer_scores(const dsa_dims *dims, const void *q_idx, const float *w_idx,
                              const void *k_idx_cache, float *scores, int64_t ld, void *stream);

/* Workspace bytes that dsa_topk_select needs for these dims (0 = none). */
DSA_API size_t dsa_topk_workspace_bytes(const dsa_dims *dims);

/*
 * dsa_topk_select -- step 2, the per-query top-k selection.
 *
 * For query i, among the causal keys j = 0 .. p_i of scores[i]: if p_i + 1 <=
 * top_k every causal key is selected; otherwise the top_k keys that come first
 * when ordered by score descending, then key index ascending, are selected
 * (a tie at the threshold goes to the lower key index; -0.0 equals +0.0).
 * idx[i] lists the selected keys in ascending order, padded with -1 to top_k.
 * The result is unique, so it is bit-exact against any correct implementation.
 * Scores must not be NaN (NaN rows give an unspecified but in-range selection).
 *
 * Arguments
 *   scores     [n_q][ld] fp32 (only the causal prefix of each row is read)
 *   idx        [n_q][top_k] int32
 *   workspace  device buffer of ws_bytes >= dsa_topk_workspace_bytes(dims) (may be NULL if 0)
 * Supports 1 <= top_k <= 2^20 and any n_q, offset.
 */
DSA_API dsa_status dsa_topk_select(const dsa_dims *dims, const float *scores, int64_t ld, int32_t *idx,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * dsa_sparse_mla_fwd -- steps 3-7, attention over the selected latent rows.
 *
 * For query i and head h, over the slots t of idx[i] whose key j = idx[i][t]
 * satisfies 0 <= j <= p_i (other slots, such as the -1 padding, are skipped):
 *   l_t        = sm_scale * sum_{d < d_latent + d_rope} q[i][h][d] * kv_cache[j][d]
 *   out[i][h]  = sum_t softmax(l)_t * kv_cache[j_t][0 : d_latent]
 *   lse[i][h]  = log(sum_t exp(l_t))          (natural log)
 * A query with no valid slot gets out = 0 and lse = -inf.
 *
 * Arguments
 *   q         [n_q][n_heads][d_latent + d_rope]   act_dtype (rotary part already applied)
 *   kv_cache  [offset + n_q][d_latent + d_rope]   act_dtype
 *   idx       [n_q][top_k] int32 (as written by dsa_topk_select, or any indices)
 *   out       [n_q][n_heads][d_latent] fp32
 *   lse       [n_q][n_heads] fp32, or NULL when not wanted
 * bf16 inputs are multiplied on the matrix cores with fp32 accumulation and an
 * fp32 softmax. Fast path: bf16 with n_heads == 64, d_latent == 512,
 * d_rope == 64, top_k a multiple of 4 (1 <= top_k <= 2^20) and a cache of
 * less than 4 GiB ((offset + n_q) * 1152 bytes); every other shape runs a
 * plain kernel (fp32 math, d_latent + d_rope <= 2048, top_k <= 4096, else
 * DSA_ERR_UNSUPPORTED).
 */
DSA_API dsa_status dsa_sparse_mla_fwd(const dsa_dims *dims, const void *q, const void *kv_cache,
                              const int32_t *idx, float *out, float *lse, void *stream);

/*
 * dsa_indexer_topk -- steps 1 and 2 fused: the top-k selection of the indexer
 * scores without the score matrix (the feedman.me page's "DSA indexer" row
 * and its per-query top-2,048 selection).
 *
 * Writes idx[n_q][top_k] exactly as dsa_indexer_scores followed by
 * dsa_topk_select would (same scores, same arithmetic, same tie rule), but
 * the indexer keeps only each query's candidates: the causal keys scoring at
 * or above a threshold taken from the query's first 2,048 keys. The select
 * then runs over those. Queries whose candidates are too few or too many
 * have their scores computed again (same arithmetic) and are selected from
 * the full row, so the result never depends on the threshold.
 *
 * Arguments as for the two calls, without the score matrix:
 *   q_idx, w_idx, k_idx_cache   as for dsa_indexer_scores
 *   idx        [n_q][top_k] int32, as for dsa_topk_select
 *   workspace  device buffer of ws_bytes >= dsa_indexer_topk_workspace_bytes(dims),
 *              16-byte aligned; contents on entry do not matter
 * The fused kernels need bf16 indexer inputs with n_idx_heads == 4, d_idx ==
 * 128, at most 65,536 cache rows and top_k <= 4,096; for other valid shapes
 * the call runs the two separate steps with the scores in the workspace.
 * dsa_indexer_topk_workspace_bytes returns 0 for invalid dims.
 */
DSA_API size_t dsa_indexer_topk_workspace_bytes(const dsa_dims *dims);
DSA_API dsa_status dsa_indexer_topk(const dsa_dims *dims, const void *q_idx, const float *w_idx,
                                    const void *k_idx_cache, int32_t *idx, void *workspace, size_t ws_bytes,
                                    void *stream);

/*
 * Decode-shaped attention: steps 3-7 for a chunk of a few queries (1-4 tokens
 * of a decode step, e.g. multi-token drafts), the decode side of the
 * feedman.me page's split (decode runs on the machine holding the cache).
 *
 * Same operation, arguments and results as dsa_sparse_mla_fwd (within fp32
 * rounding: the order of the softmax sums differs). On the fast path each
 * query's index row is split into slices of whole 32-slot tiles that run on
 * separate workgroups; their normalised partial outputs and log-sum-exps are
 * merged by a second kernel. The partials live in the caller's workspace:
 *   workspace  device buffer of ws_bytes >= dsa_sparse_mla_decode_workspace_bytes(dims),
 *              16-byte aligned (may be NULL when that size is 0: no split)
 * dsa_sparse_mla_decode_workspace_bytes returns 0 for dims that need no split
 * (many queries, or the plain kernel) and for invalid dims.
 */
DSA_API size_t dsa_sparse_mla_decode_workspace_bytes(const dsa_dims *dims);
DSA_API dsa_status dsa_sparse_mla_decode(const dsa_dims *dims, const void *q, const void *kv_cache,
                                         const int32_t *idx, float *out, float *lse, void *workspace,
                                         size_t ws_bytes, void *stream);

/*
 * dsa_sparse_mla_decode_noalloc -- dsa_sparse_mla_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same operation, arguments and results as dsa_sparse_mla_decode with the
 * workspace removed: the split partials go to a scratch array the library
 * holds in device memory, 32 MiB on each GPU it runs on, kept until the
 * process ends. Nothing is allocated or freed by this call. The scratch is
 * that of the current device (the stream must belong to it); every call on a
 * GPU shares it, so calls that overlap in time on one GPU race and must be
 * ordered by the caller (one stream, or events). Nothing in it needs to start
 * at zero: each call writes every partial it reads.
 *
 * Returns DSA_ERR_WORKSPACE, before anything is enqueued, when the partials
 * would exceed the scratch (dsa_sparse_mla_decode_workspace_bytes(dims) >
 * 32 MiB: more than 255 split partials of 64 heads x 513 fp32, e.g. more
 * than 15 queries at 16 splits of a 2,048-slot index row); calls that need no
 * split (dsa_sparse_mla_decode_workspace_bytes(dims) == 0) never touch it.
 */
DSA_API dsa_status dsa_sparse_mla_decode_noalloc(const dsa_dims *dims, const void *q, const void *kv_cache,
                                                 const int32_t *idx, float *out, float *lse, void *stream);

/*
 * dsa_prefill_chunk -- one chunk of a chunked prefill: the cache append that
 * precedes the hot path, then steps 1-7.
 *
 * A prompt is processed as successive chunks (the feedman.me page profiles
 * 8,192 tokens in 2,048-token chunks, and a 17.5k-token prompt). For the
 * chunk at rows [offset, offset + n_q) this call
 *   1. copies kv_chunk   [n_q][d_latent + d_rope] act_dtype into kv_cache[offset ..],
 *             k_idx_chunk [n_q][d_idx]           idx_dtype into k_idx_cache[offset ..]
 *      (no copy when a chunk pointer already equals its destination);
 *   2. runs dsa_indexer_scores, dsa_topk_select and dsa_sparse_mla_fwd on the
 *      chunk, with the arguments and results documented above.
 * Because every query's results depend only on its own row of inputs and on
 * the cache rows it can see, the outputs of a query are bit-identical however
 * the prompt is split into chunks.
 *
 * Arguments as for the three calls, plus
 *   kv_chunk, k_idx_chunk  the chunk's new cache rows (device, 16-byte aligned;
 *                          must not partially overlap their destination)
 *   kv_cache, k_idx_cache  caches with room for offset + n_q rows
 *   scores     as for dsa_indexer_scores, or NULL: steps 1 and 2 then run as
 *              dsa_indexer_topk (same indices, no score matrix; `ld` is
 *              ignored) with `workspace` of ws_bytes >=
 *              dsa_indexer_topk_workspace_bytes(dims). On MI355X that is the
 *              faster way once the context reaches about 32k keys; below it
 *              the two calls are as fast or faster.
 *   workspace, ws_bytes  as for dsa_topk_select (which needs none), or the
 *              fused call's workspace when scores is NULL
 * Every argument of the three steps is validated before anything is enqueued.
 */
DSA_API dsa_status dsa_prefill_chunk(const dsa_dims *dims, const void *q, const void *kv_chunk,
                                     const void *q_idx, const float *w_idx, const void *k_idx_chunk,
                                     void *kv_cache, void *k_idx_cache, float *scores, int64_t ld,
                                     int32_t *idx, float *out, float *lse, void *workspace,
                                     size_t ws_bytes, void *stream);

/*
 * dsa_self_test -- the matrix-core layout self-test on the current device.
 *
 * Runs known small-integer products through each matrix-core instruction form
 * and operand path the fast kernels use (register operands of the 16x16x32
 * and 32x32x16 bf16 forms, and the transposing LDS read that feeds the value
 * operand of attention) and compares every result with the exact product
 * computed on the host. A layout other than the one the kernels assume (for
 * example a transposed operand) fails it. Prompted by TensorFold issue #743,
 * "Proposal: restore single-Mac GLM-5.3-Flash on the M3 Ultra", which asks
 * for a load-time fragment-layout check that catches a transposed operand.
 *
 * Synchronous; runs once per device (later calls return the cached result).
 * Every other call runs it before its first launch on a device, unless its
 * stream is being captured into a graph: call this function before capturing.
 * Returns DSA_OK, or DSA_ERR_DEVICE when a product is wrong or HIP fails.
 */
DSA_API dsa_status dsa_self_test(void);

/* Static description of a status code (never NULL). */
DSA_API const char *dsa_status_string(dsa_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
DSA_API int32_t dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
