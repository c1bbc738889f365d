// fused.hip -- steps 1 and 2 without the score matrix: the indexer writes only
// the keys each query could select, and the top-k select runs over those.
//
// The result is that of dsa_indexer_scores followed by dsa_topk_select (the
// feedman.me page, per-component profile row "DSA indexer", and the top-2,048
// selection of the paragraph on the work that is not a matmul). Four launches:
//   sample  : the indexer over each query's first 2,048 keys (the regular MFMA
//             kernel, into a small [n_q][2048] buffer);
//   tau     : per query, the threshold tau those keys give (their key of rank
//             a fifth above where the k-th key is expected, plus 16, to 22
//             bits; the same rule as the filtered select over a score row);
//   filter  : the indexer over every key in candidate mode: each causal score
//             whose key is >= tau is written with its key index, in key order,
//             to the query's segment of the key range (no score matrix);
//   select  : per query, the candidates of its segments are gathered into LDS
//             in key order and selected exactly (as over a score row's
//             candidates). If there are fewer than k of them (tau too high)
//             or more than fit in LDS, the query's scores are computed again
//             with the same matrix-core instruction sequence as the indexer
//             (so the same values) into its segment area, and the row is
//             selected without a threshold.
#include "common.h"
#include "device_checks.h"
#include "kernels.h"
#include "select_common.h"

namespace dsa {

namespace {

constexpr int kMaxUnits = 2 * kFsThreads;  // key ranges of one query: 65,536 keys / 128
static_assert(kFusedMaxRow == kFsMaxRow && kFusedMaxTopk == kFsCap && kFusedSample == kFsSample,
              "the workspace layout's limits are the select's");
static_assert(kFusedMaxRow / 128 <= kMaxUnits, "a query's key ranges fit the offsets array");

// Threshold of each query with more than k causal keys, from the scores of
// its first min(n, 2048) keys (sample row i, 2048 floats a row).
__global__ __launch_bounds__(kFsThreads) void tau_kernel(int offset, int k, const float* __restrict__ sample,
                                                         uint32_t* __restrict__ tau_out, float* __restrict__ tf_out) {
  lds_poison();
  __shared__ FsSmem sm;
  int buf = 0;
  const int i = blockIdx.x;
  const int n = offset + i + 1;
  if (n <= k) return;  // every causal key is selected: no threshold
  const float* __restrict__ row = sample + static_cast<int64_t>(i) * kFsSample;
  const int S = min(n, kFsSample);
  f32x4 cur[kFsSampleSlices];
#pragma unroll
  for (int s = 0; s < kFsSampleSlices; ++s) cur[s] = fs_load4(row, s * kFsSlice, S);
  fs_zero<true>(sm.hist);
  fs_zero<false>(sm.ckey);
  lds_sync();
  const uint32_t tau = fs_sample_tau(sm, buf, cur, n, k);
  if (threadIdx.x == 0) {
    tau_out[i] = tau;
    tf_out[i] = key_to_score(tau);
  }
}

// The scores of query i's first n keys, computed as the indexer computes them
// (32x32x16 bf16 products over the 128 dims in the same k-step order, then
// the ReLU / weight / head sum in the same order), into row[0 .. n). The
// query's 4 heads are rows 0..3 of the A operand; each wave takes 32 keys.
__device__ __forceinline__ void rescore_row(int i, int n, int t_ctx, const uint16_t* __restrict__ q_idx,
                                            const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
                                            float* __restrict__ row) {
  constexpr int D = 128, KS = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  bf16x8 a[KS];
  {
    const uint16_t* src = q_idx + (static_cast<int64_t>(i) * 4 + (l32 & 3)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = l32 < 4 ? *reinterpret_cast<const u32x4*>(src + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
      a[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float wh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wh[h] = w[static_cast<int64_t>(i) * 4 + h];
  for (int nb = 32 * wave; nb < n; nb += 32 * (kFsThreads / kWave)) {
    const int key = nb + l32;
    const int krow = key < t_ctx ? key : t_ctx - 1;
    const uint16_t* bsrc = k_idx + static_cast<int64_t>(krow) * D + 8 * hi;
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bsrc + 16 * ks));
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], acc, 0, 0, 0);
    // register h of a lane of the lower half: A row h (head h) at key nb + l32
    float sc = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) sc = fmaf(wh[h], __int_as_float(max(__float_as_int(acc[h]), 0)), sc);
    sc = sc + 0.0f;
    if (hi == 0 && key < n) row[key] = sc;
  }
}

// Per query: its candidates (the segments of the key ranges holding causal
// keys) into LDS in key order, then the exact select over them; the rescore
// fallback when they are fewer than k or do not fit.
__global__ __launch_bounds__(kFsThreads) void cand_select_kernel(int offset, int n_q, int k, IndexerCandidates fo,
                                                                 int keys_per_unit, const uint32_t* __restrict__ tau,
                                                                 const uint16_t* __restrict__ q_idx,
                                                                 const float* __restrict__ w,
                                                                 const uint16_t* __restrict__ k_idx,
                                                                 int32_t* __restrict__ idx) {
  lds_poison();
  __shared__ FsSmem sm;
  __shared__ uint32_t uoff[kMaxUnits + 1];
  int buf = 0;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int n = offset + i + 1;
  int32_t* __restrict__ out = idx + static_cast<int64_t>(i) * k;
  if (n <= k) {
    for (int t = tid; t < k; t += kFsThreads) out[t] = t < n ? t : -1;
    return;
  }
  const int nu = (n - 1) / keys_per_unit + 1;  // key ranges with causal keys (<= kMaxUnits: checked on the host)
  const int32_t* __restrict__ cnt = fo.counts + static_cast<int64_t>(i) * fo.n_kr;
  const uint32_t c0 = 2 * tid < nu ? static_cast<uint32_t>(cnt[2 * tid]) : 0u;
  const uint32_t c1 = 2 * tid + 1 < nu ? static_cast<uint32_t>(cnt[2 * tid + 1]) : 0u;
  fs_zero<true>(sm.hist);
  if (tid == 0) {
    sm.low_or = 0u;
    sm.low_and = 0x3FFu;
  }
  uint64_t total;
  const uint32_t before = static_cast<uint32_t>(fs_scan(c0 + c1, &total, sm, buf));
  const uint32_t m = static_cast<uint32_t>(total);
  if (2 * tid < nu) uoff[2 * tid] = before;
  if (2 * tid + 1 < nu) uoff[2 * tid + 1] = before + c0;
  if (tid == 0) uoff[nu] = m;
  const int64_t seg0 = static_cast<int64_t>(i) * fo.row_cap;
  if (m >= static_cast<uint32_t>(k) && m <= static_cast<uint32_t>(kFsCap)) {
    __syncthreads();
    // Each wave copies segments u and u + 4 (of every eighth pair) to their
    // offsets, up to four candidates of each per lane in flight.
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int kWaves = kFsThreads / kWave;
    for (int u0 = wave; u0 < nu; u0 += 2 * kWaves) {
      uint32_t o[2], c[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = u0 + h * kWaves;
        o[h] = u < nu ? uoff[u] : 0u;
        c[h] = u < nu ? uoff[u + 1] - o[h] : 0u;
      }
      const uint32_t cmax = max(c[0], c[1]);
      for (uint32_t e0 = 0; e0 < cmax; e0 += 4 * kWave) {  // wave-uniform
        uint2 v[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t e = e0 + lane + r * kWave;
            const int64_t src = seg0 + static_cast<int64_t>(u0 + h * kWaves) * keys_per_unit + e;
            v[h][r] = e < c[h] ? fo.cand[src] : uint2{0u, 0u};
          }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t e = e0 + lane + r * kWave;
            if (e < c[h]) {
              sm.ckey[o[h] + e] = v[h][r].x;
              sm.cidx[o[h] + e] = static_cast<uint16_t>(v[h][r].y);
            }
          }
      }
    }
    __syncthreads();
    fs_select_candidates(sm, buf, nullptr, n, k, out, tau[i], static_cast<int>(m));
    return;
  }
  // fallback: the query's scores again, into its segment area, and the select
  // of that row without a threshold
  float* __restrict__ row = reinterpret_cast<float*>(fo.cand + seg0);  // 2 * row_cap floats
  rescore_row(i, n, offset + n_q, q_idx, w, k_idx, row);
  __threadfence();
  __syncthreads();
  fs_select_row(sm, buf, row, n, k, out);
}

hipError_t check_fused_kernels_now() {
  const void* ks[] = {reinterpret_cast<const void*>(tau_kernel), reinterpret_cast<const void*>(cand_select_kernel)};
  for (const void* k : ks) {
    const hipError_t e = check_launch_limits(k, kFsThreads, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t check_fused_kernels() {
  static PerDeviceCache cache;
  return once_per_device(cache, check_fused_kernels_now);
}

hipError_t launch_indexer_topk(const IndexerArgs& ia, const TopkArgs& ta, const FusedLayout& L, void* workspace,
                               hipStream_t s) {
  if (ia.n_q == 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (!L.fused) {
    // scores into the workspace, then the select over them
    IndexerArgs a = ia;
    a.scores = reinterpret_cast<float*>(ws + L.scores_off);
    a.ld = L.scores_ld;
    TopkArgs t = ta;
    t.scores = a.scores;
    t.ld = L.scores_ld;
    hipError_t e = launch_indexer(a, s);
    return e != hipSuccess ? e : launch_topk(t, s);
  }
  uint32_t* tau = reinterpret_cast<uint32_t*>(ws + L.tau_off);
  float* tf = reinterpret_cast<float*>(ws + L.tf_off);
  float* sample = reinterpret_cast<float*>(ws + L.sample_off);
  IndexerCandidates fo{tf,
                       reinterpret_cast<uint2*>(ws + L.cand_off),
                       reinterpret_cast<int32_t*>(ws + L.counts_off),
                       L.row_cap,
                       L.n_kr,
                       ta.top_k};
  // 1. scores of every query's first kFsSample keys (causally masked)
  IndexerArgs sa = ia;
  sa.scores = sample;
  sa.ld = kFsSample;
  hipError_t e = launch_indexer(sa, s);
  // 2. thresholds
  if (e == hipSuccess)
    e = launch_kernel(tau_kernel, dim3(ia.n_q), dim3(kFsThreads), 0, s, ia.offset, ta.top_k,
                      static_cast<const float*>(sample), tau, tf);
  // 3. candidates
  IndexerArgs ca = ia;
  ca.ld = static_cast<int64_t>(ia.offset) + ia.n_q;
  if (e == hipSuccess) e = launch_indexer_candidates(ca, fo, s);
  // 4. select
  if (e == hipSuccess)
    e = launch_kernel(cand_select_kernel, dim3(ia.n_q), dim3(kFsThreads), 0, s, ia.offset, ia.n_q, ta.top_k, fo,
                      L.keys_per_unit, static_cast<const uint32_t*>(tau), static_cast<const uint16_t*>(ia.q_idx),
                      ia.w, static_cast<const uint16_t*>(ia.k_idx), ta.idx);
  return e;
}

}  // namespace dsa
