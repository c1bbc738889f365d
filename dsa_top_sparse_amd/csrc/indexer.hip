// indexer.hip -- step 1 of the DSA prefill path: indexer scores.
//
// For query i (absolute position p = offset + i) and key j:
//   s[i][j] = sum_h w[i][h] * max(0, <q_idx[i][h], k_idx[j]>)   for j <= p,
//   s[i][j] = -inf                                               for p < j < ld.
// (feedman.me page, per-component profile row "DSA indexer"; the formula is
// this library's reading, the pages print none.)
//
// Fast kernel (bf16, 4 indexer heads): one dense contraction on the matrix
// cores. Rows of the A operand are (query, head) pairs laid out as 4*q + h, so
// in the 32x32 MFMA result each lane holds the 4 head dot products of one
// (query, key) pair and the ReLU / weight / head sum happens in registers.
// With d_idx = 128 (indexer_lds_kernel) the scores of a wave's 8 queries x
// 32 keys pass through a small LDS tile and leave as 16-byte stores (4
// consecutive keys of one query per lane); the other widths store one fp32
// score per lane, 32 lanes covering 32 consecutive keys of one query row.
#include "common.h"
#include "device_checks.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kIdxThreads = 256;   // 4 waves
constexpr int kIdxQueries = 64;    // queries per workgroup (16 per wave)
constexpr int kIdxHeads = 4;

__device__ __forceinline__ float plain_load(const float* p, int64_t e) { return p[e]; }
__device__ __forceinline__ float plain_load(const uint16_t* p, int64_t e) { return bf16_to_f32(p[e]); }

// Any dtype / head count / width. grid = (ceil(ld / 256), n_q).
template <typename T>
__global__ __launch_bounds__(256) void indexer_plain_kernel(int n_q, int offset, int n_heads,
                                                            int d_idx, const T* __restrict__ q_idx,
                                                            const float* __restrict__ w,
                                                            const T* __restrict__ k_idx,
                                                            float* __restrict__ scores, int64_t ld) {
  lds_poison(4u * (uint32_t)(n_heads * d_idx));  // sq[]
  extern __shared__ float sq[];  // [n_heads][d_idx] of this query
  const int i = blockIdx.y;
  const int hd = n_heads * d_idx;
  for (int e = threadIdx.x; e < hd; e += blockDim.x) sq[e] = plain_load(q_idx, (int64_t)i * hd + e);
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= ld) return;
  const int64_t p = (int64_t)offset + i;
  float out = -INFINITY;
  if (j <= p) {
    float s = 0.0f;
    for (int h = 0; h < n_heads; ++h) {
      float dot = 0.0f;
      for (int d = 0; d < d_idx; ++d) dot = fmaf(sq[h * d_idx + d], plain_load(k_idx, j * d_idx + d), dot);
      s = fmaf(w[(int64_t)i * n_heads + h], fmaxf(dot, 0.0f), s);
    }
    out = (s == 0.0f) ? 0.0f : s;  // +0.0, never -0.0
  }
  scores[(int64_t)i * ld + j] = out;
}

// Fill scores[rows q0 .. q0+nrows)[k0 .. k1) with -inf (fully non-causal range).
__device__ __forceinline__ void fill_neg_inf(float* __restrict__ scores, int64_t ld, int q0, int nrows,
                                             int64_t k0, int64_t k1) {
  const int width = (int)(k1 - k0);
  for (int r = 0; r < nrows; ++r) {
    float* row = scores + (int64_t)(q0 + r) * ld + k0;
    for (int c = threadIdx.x; c < width; c += (int)blockDim.x) __builtin_nontemporal_store(-INFINITY, row + c);
  }
}

// Work unit of workgroup bid: (key range kr of keys_per_unit keys, 64-query
// block qb); false if the workgroup has none. Workgroups reach the 8 XCDs in
// turn (XCD = bid % 8). With a multiple of 8 query blocks, XCD x takes the
// query blocks qb = x (mod 8) of every key range, latest (most causal keys)
// first, and visits the key ranges from x * n_kr / 8 on. Every XCD then gets
// the same share of the causal work (a contiguous run of units per XCD left
// the XCDs holding the early key ranges with a third more work than the mean
// on an 8k chunk at an 8k offset), each XCD holds only a few key ranges in
// its L2 at a time, and the workgroups resident on the chip write into all key
// ranges of their score rows at once instead of a narrow band of columns.
// Otherwise XCD x takes a contiguous run of units.
__device__ __forceinline__ bool unit_of(int bid, int n_qb, int n_units, int units_per_xcd, int& kr, int& qb) {
  if ((n_qb & 7) == 0) {
    const int x = bid & 7, k = bid >> 3, per = n_qb >> 3;
    const int n_kr = n_units / n_qb;
    const int jr = k / per, i = k - jr * per;
    if (jr >= n_kr) return false;
    kr = (jr + x * (n_kr >> 3)) % n_kr;
    qb = 8 * (per - 1 - i) + x;
    return true;
  }
  const int u = (bid & 7) * units_per_xcd + (bid >> 3);
  if (u >= n_units) return false;
  kr = u / n_qb;
  qb = u - kr * n_qb;
  return true;
}

// bf16, 4 indexer heads, d_idx = D (multiple of 16).
// Work unit = (64-query block, range of `keys_per_unit` keys), see unit_of.
template <int D>
__global__ __launch_bounds__(kIdxThreads) void indexer_mfma_kernel(
    int n_q, int offset, const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, float* __restrict__ scores, int64_t ld, int n_qb,
    int n_units, int units_per_xcd, int keys_per_unit) {
  lds_poison();
  constexpr int KS = D / 16;  // k-steps of the 32x32x16 MFMA
  int kr, qb;
  if (!unit_of((int)blockIdx.x, n_qb, n_units, units_per_xcd, kr, qb)) return;
  const int q0 = qb * kIdxQueries;
  const int nrows = min(kIdxQueries, n_q - q0);
  const int64_t k_begin = (int64_t)kr * keys_per_unit;
  const int64_t k_end = min<int64_t>(ld, k_begin + keys_per_unit);
  const int64_t t_ctx = (int64_t)offset + n_q;
  const int64_t p_max = (int64_t)offset + q0 + nrows - 1;
  if (k_begin > p_max) {  // every key of the range lies beyond every query of the block
    fill_neg_inf(scores, ld, q0, nrows, k_begin, k_end);
    return;
  }

  __shared__ float sw[kIdxQueries][kIdxHeads];
  for (int e = threadIdx.x; e < kIdxQueries * kIdxHeads; e += kIdxThreads) {
    const int q = e >> 2;
    sw[q][e & 3] = (q < nrows) ? w[(int64_t)(q0 + q) * kIdxHeads + (e & 3)] : 0.0f;
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // A operand: rows (query, head) = 4*q + h of this wave's 16 queries, two
  // 32-row blocks. Lane holds row l32, k-slice 8*hi .. 8*hi+7 of each k-step.
  bf16x8 a[2][KS];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int qrow = wave * 16 + mb * 8 + (l32 >> 2);  // query within the block
    const bool ok = qrow < nrows;
    const uint16_t* src = q_idx + ((int64_t)(q0 + (ok ? qrow : 0)) * kIdxHeads + (l32 & 3)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(src + 16 * ks) : u32x4{0, 0, 0, 0};
      a[mb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();

  for (int64_t nb = k_begin; nb < k_end; nb += 32) {
    const int64_t key = nb + l32;
    if (nb > p_max) {  // whole 32-key block is beyond the causal frontier
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qrow = wave * 16 + mb * 8 + 2 * g + hi;
          if (qrow < nrows && key < k_end)
            __builtin_nontemporal_store(-INFINITY, scores + (int64_t)(q0 + qrow) * ld + key);
        }
      continue;
    }
    // B operand: key row (clamped into the cache; clamped keys are masked).
    const int64_t krow = key < t_ctx ? key : t_ctx - 1;
    const uint16_t* bsrc = k_idx + krow * D + 8 * hi;
    bf16x8 b[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bsrc + 16 * ks));
    f32x16 acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      acc[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb][ks], b[ks], acc[mb], 0, 0, 0);
    }
    // Result layout: register r of lane (l32, hi) holds row 8*(r/4) + 4*hi + r%4
    // = 4*query + head with query = 2*(r/4) + hi and head = r%4, column l32.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qrow = wave * 16 + mb * 8 + 2 * g + hi;
        if (qrow < nrows && key < k_end) {
          float s = 0.0f;
#pragma unroll
          for (int h = 0; h < 4; ++h) s = fmaf(sw[qrow][h], fmaxf(acc[mb][4 * g + h], 0.0f), s);
          s = (s == 0.0f) ? 0.0f : s;
          const int64_t p = (int64_t)offset + q0 + qrow;
          __builtin_nontemporal_store(key <= p ? s : -INFINITY, scores + (int64_t)(q0 + qrow) * ld + key);
        }
      }
  }
}


// d_idx = 128: 8 waves of 8 queries each (one 32-row A block, 32 q_idx
// registers per wave, so that four waves fit per SIMD). The keys of a stage
// (64 rows x 256 B) are read from global memory once per workgroup and shared
// by its 8 waves through LDS (double buffered; the next stage's loads are in
// flight during this stage's MFMAs), instead of every wave reading them from
// L2. A key row's 16-byte piece s is stored at position s ^ (row & 15), so the
// B-operand reads (16 consecutive key rows, one piece each) hit all 64 banks.
constexpr int kIdxStageKeys = 64;
constexpr int kIdxRowBytes = 256;  // 128 bf16
constexpr int kIdx8Threads = 512;  // indexer_lds_kernel: 8 waves of 8 queries
constexpr int kTbRow = 36;         // floats per row of a wave's score tile (32 keys + pad)

// FILTER: instead of the score matrix, every causal score >= the query's
// threshold is written with its key index to the query's candidate segment of
// this key range (in key order, at most keys_per_unit of them), and the count
// per (query, key range) to counts; the scores are the same, computed the
// same way. Queries with no more causal keys than top_k write nothing.
template <bool FILTER>
__global__ __launch_bounds__(kIdx8Threads) __attribute__((amdgpu_waves_per_eu(4))) void indexer_lds_kernel(
    int n_q, int offset, const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ k_idx, float* __restrict__ scores, int64_t ld, int n_qb,
    int n_units, int units_per_xcd, int keys_per_unit, IndexerCandidates fo) {
  lds_poison();
  constexpr int D = 128, KS = D / 16;
  int kr, qb;
  if (!unit_of((int)blockIdx.x, n_qb, n_units, units_per_xcd, kr, qb)) return;
  const int q0 = qb * kIdxQueries;
  const int nrows = min(kIdxQueries, n_q - q0);
  const int64_t k_begin = (int64_t)kr * keys_per_unit;
  const int64_t k_end = min<int64_t>(ld, k_begin + keys_per_unit);
  const int64_t t_ctx = (int64_t)offset + n_q;
  const int64_t p_max = (int64_t)offset + q0 + nrows - 1;
  if (k_begin > p_max) {  // every key of the range lies beyond every query of the block
    if (!FILTER) fill_neg_inf(scores, ld, q0, nrows, k_begin, k_end);
    return;
  }
  // keys [k_begin, k_comp) need the product; [k_comp, k_end) are past every query
  const int64_t k_comp = min<int64_t>(k_end, p_max + 1);
  const int n_stages = (int)((k_comp - k_begin + kIdxStageKeys - 1) / kIdxStageKeys);

  __shared__ float sw[kIdxQueries][kIdxHeads];
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kIdxStageKeys * kIdxRowBytes];
  __shared__ __attribute__((aligned(16))) float tbuf[kIdx8Threads / 64][8 * kTbRow];
  const bool vec_ok = (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  for (int e = threadIdx.x; e < kIdxQueries * kIdxHeads; e += kIdx8Threads) {
    const int q = e >> 2;
    sw[q][e & 3] = (q < nrows) ? w[(int64_t)(q0 + q) * kIdxHeads + (e & 3)] : 0.0f;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets wave-level tests branch on scalars
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Stage loads: thread t copies pieces 2 (t % 8), +1 of key row t / 8.
  const int ld_row = tid >> 3, ld_p0 = 2 * (tid & 7);
  auto load_stage = [&](int st, u32x4 (&v)[2]) {
    const int64_t key = k_begin + (int64_t)st * kIdxStageKeys + ld_row;
    const int64_t krow = key < t_ctx ? key : t_ctx - 1;  // clamped rows are masked later
    const u32x4* src = reinterpret_cast<const u32x4*>(k_idx + krow * D) + ld_p0;
#pragma unroll
    for (int x = 0; x < 2; ++x) v[x] = src[x];
  };
  auto store_stage = [&](int buf, const u32x4 (&v)[2]) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
      *reinterpret_cast<u32x4*>(&kbuf[buf][ld_row * kIdxRowBytes + 16 * ((ld_p0 + x) ^ (ld_row & 15))]) = v[x];
  };

  // A operand: rows (query, head) = 4*q + h of this wave's 8 queries, one
  // 32-row block. Lane holds row l32, k-slice 8*hi .. 8*hi+7 of each k-step.
  bf16x8 a[1][KS];
#pragma unroll
  for (int mb = 0; mb < 1; ++mb) {
    const int qrow = wave * 8 + (l32 >> 2);
    const bool ok = qrow < nrows;
    const uint16_t* src = q_idx + ((int64_t)(q0 + (ok ? qrow : 0)) * kIdxHeads + (l32 & 3)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(src + 16 * ks) : u32x4{0, 0, 0, 0};
      a[mb][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // FILTER: per query pair g (queries 2 g and 2 g + 1 of the wave's eight,
  // held by the lower and the upper half-wave) the two thresholds (+inf where
  // nothing is written), segment offsets and running counts, all wave-uniform.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  float tf_lo[4], tf_hi[4];
  uint32_t seg_lo[4], seg_hi[4], cnt_lo[4] = {0u, 0u, 0u, 0u}, cnt_hi[4] = {0u, 0u, 0u, 0u};
  if (FILTER) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = wave_u * 8 + 2 * g;
      tf_lo[g] = (r0 < nrows && (int64_t)offset + q0 + r0 + 1 > fo.top_k) ? fo.tf[q0 + r0] : INFINITY;
      tf_hi[g] = (r0 + 1 < nrows && (int64_t)offset + q0 + r0 + 2 > fo.top_k) ? fo.tf[q0 + r0 + 1] : INFINITY;
      seg_lo[g] = static_cast<uint32_t>((int64_t)(q0 + r0) * fo.row_cap + (int64_t)kr * keys_per_unit);
      seg_hi[g] = seg_lo[g] + static_cast<uint32_t>(fo.row_cap);
    }
  }
  u32x4 pre[2];
  load_stage(0, pre);
  store_stage(0, pre);
  __syncthreads();

  for (int st = 0; st < n_stages; ++st) {
    const bool more = st + 1 < n_stages;
    if (more) load_stage(st + 1, pre);  // in flight during this stage
    const uint8_t* kb = kbuf[st & 1];
#pragma unroll
    for (int sub = 0; sub < kIdxStageKeys / 32; ++sub) {
      const int64_t nb = k_begin + (int64_t)st * kIdxStageKeys + 32 * sub;
      if (nb >= k_comp) break;  // block-uniform
      const int64_t key = nb + l32;
      const int krow = 32 * sub + l32;
      bf16x8 b[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        b[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               &kb[krow * kIdxRowBytes + 16 * ((2 * ks + hi) ^ (krow & 15))]));
      f32x16 acc[1];
#pragma unroll
      for (int mb = 0; mb < 1; ++mb) {
        acc[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb][ks], b[ks], acc[mb], 0, 0, 0);
      }
      // register r of lane (l32, hi): query 2 (r / 4) + hi of the 8-query group, head r % 4, key l32.
      // ReLU as an integer max on the bits (one instruction: a negative float is a
      // negative int32). No score comes out as -0: the head sum starts as
      // fma(w, x, +0), and under round-to-nearest an exactly zero sum of
      // nonzero terms, or of zeros of both signs, is +0 (fp32 denormals are
      // kept, so no tiny result flushes to -0). The causal mask is
      // needed only where the block reaches the wave's first query
      // (wave-uniform test).
      if (FILTER) {
        // the lane's causal scores >= its query's threshold, in key order,
        // to that query's segment of this key range
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qrow = wave * 8 + 2 * g + hi;
          float sc = 0.0f;
#pragma unroll
          for (int h = 0; h < 4; ++h)
            sc = fmaf(sw[qrow][h], __int_as_float(max(__float_as_int(acc[0][4 * g + h]), 0)), sc);
          const bool keep = key <= (int64_t)offset + q0 + qrow && sc >= (hi ? tf_hi[g] : tf_lo[g]);
          const uint64_t m = __ballot(keep);
          const uint32_t m_lo = static_cast<uint32_t>(m), m_hi = static_cast<uint32_t>(m >> 32);
          if (keep) {
            const uint32_t at = (hi ? seg_hi[g] + cnt_hi[g] : seg_lo[g] + cnt_lo[g]) +
                                __builtin_popcount((hi ? m_hi : m_lo) & ((1u << l32) - 1u));
            fo.cand[at] = uint2{__float_as_uint(sc), static_cast<uint32_t>(key)};
          }
          cnt_lo[g] += __builtin_popcount(m_lo);
          cnt_hi[g] += __builtin_popcount(m_hi);
        }
        continue;
      }
      const bool all_causal = nb + 31 <= (int64_t)offset + q0 + wave * 8;
      const bool all_in = nb + 32 <= k_end && q0 + wave * 8 + 8 <= n_q;  // every row and key of the sub-block exists
      if (vec_ok && all_in) {
        // Through this wave's LDS tile, so that the stores are 16-byte vectors
        // (4 keys of one query per lane) instead of one score per lane.
        float* tb = tbuf[wave];
        // Score of row qr (of the wave's 8 queries) for the lane's key.
        auto head_sum = [&](int g, int qr) {
          float sc = 0.0f;
#pragma unroll
          for (int h = 0; h < 4; ++h)
            sc = fmaf(sw[wave * 8 + qr][h], __int_as_float(max(__float_as_int(acc[0][4 * g + h]), 0)), sc);
          return sc;
        };
        if (all_causal) {
#pragma unroll
          for (int g = 0; g < 4; ++g) tb[(2 * g + hi) * kTbRow + l32] = head_sum(g, 2 * g + hi);
        } else {
          // key nb + l32 is causal for row qr iff l32 + rel <= qr; here
          // -32 < rel < 64 (the sub-block reaches the wave's first query and
          // starts at or before the block's last one)
          const int rel = (int)(nb - ((int64_t)offset + q0 + wave * 8));
          const int lk = l32 + rel;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int qr = 2 * g + hi;
            const float sc = head_sum(g, qr);
            tb[qr * kTbRow + l32] = lk <= qr ? sc : -INFINITY;
          }
        }
#pragma unroll
        for (int x = 0; x < 1; ++x) {
          const int piece = 64 * x + lane, r = piece >> 3, c = piece & 7;
          const f32x4 v = *reinterpret_cast<const f32x4*>(&tb[r * kTbRow + 4 * c]);
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(scores + (int64_t)(q0 + wave * 8 + r) * ld + nb + 4 * c));
        }
        continue;
      }
#pragma unroll
      for (int mb = 0; mb < 1; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qrow = wave * 8 + 2 * g + hi;
          if (all_in || (qrow < nrows && key < k_end)) {
            float sc = 0.0f;
#pragma unroll
            for (int h = 0; h < 4; ++h)
              sc = fmaf(sw[qrow][h], __int_as_float(max(__float_as_int(acc[mb][4 * g + h]), 0)), sc);
            if (!all_causal) {
              const int64_t p = (int64_t)offset + q0 + qrow;
              sc = key <= p ? sc : -INFINITY;
            }
            __builtin_nontemporal_store(sc, scores + (int64_t)(q0 + qrow) * ld + key);
          }
        }
    }
    if (more) {
      store_stage((st + 1) & 1, pre);  // the other buffer: its last readers finished before the previous barrier
      __syncthreads();
    }
  }
  if (FILTER) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qrow = wave * 8 + 2 * g + hi;
      if (l32 == 0 && qrow < nrows)
        fo.counts[(int64_t)(q0 + qrow) * fo.n_kr + kr] = static_cast<int32_t>(hi ? cnt_hi[g] : cnt_lo[g]);
    }
    return;
  }
  // Keys past every query of the block: the 32-key blocks above wrote up to
  // the first multiple of 32 at or after k_comp (masked to -inf per row).
  const int64_t written = min<int64_t>(k_end, k_begin + 32 * ((k_comp - k_begin + 31) / 32));
  if (written < k_end) fill_neg_inf(scores, ld, q0, nrows, written, k_end);
}


template <int D>
hipError_t launch_mfma(const IndexerArgs& a, hipStream_t s) {
  const IndexerUnits un = indexer_units(a.n_q, a.ld);
  const int n_qb = un.n_qb;
  const int64_t kpu = un.keys_per_unit;
  const int64_t n_kr = un.n_kr;
  const int64_t n_units = n_kr * n_qb;
  if (n_units > (int64_t)1 << 30) return hipErrorInvalidValue;
  const int units_per_xcd = (int)((n_units + 7) / 8);
  const int grid = units_per_xcd * 8;
  if (D == 128 && kpu % kIdxStageKeys == 0)
    return launch_kernel(indexer_lds_kernel<false>, dim3(grid), dim3(kIdx8Threads), 0, s, a.n_q, a.offset,
                         static_cast<const uint16_t*>(a.q_idx), a.w, static_cast<const uint16_t*>(a.k_idx), a.scores,
                         a.ld, n_qb, (int)n_units, units_per_xcd, (int)kpu, IndexerCandidates{});
  return launch_kernel(indexer_mfma_kernel<D>, dim3(grid), dim3(kIdxThreads), 0, s, a.n_q, a.offset,
                       static_cast<const uint16_t*>(a.q_idx), a.w, static_cast<const uint16_t*>(a.k_idx), a.scores,
                       a.ld, n_qb, (int)n_units, units_per_xcd, (int)kpu);
}

hipError_t check_indexer_kernels_now() {
  const struct {
    const void* fn;
    int threads;
    size_t dyn_lds;
  } ks[] = {
      {reinterpret_cast<const void*>(indexer_lds_kernel<false>), kIdx8Threads, 0},
      {reinterpret_cast<const void*>(indexer_lds_kernel<true>), kIdx8Threads, 0},
      {reinterpret_cast<const void*>(indexer_mfma_kernel<32>), kIdxThreads, 0},
      {reinterpret_cast<const void*>(indexer_mfma_kernel<64>), kIdxThreads, 0},
      {reinterpret_cast<const void*>(indexer_mfma_kernel<128>), kIdxThreads, 0},
      {reinterpret_cast<const void*>(indexer_mfma_kernel<256>), kIdxThreads, 0},
      {reinterpret_cast<const void*>(indexer_plain_kernel<uint16_t>), 256, sizeof(float) * kPlainIndexerMaxElems},
      {reinterpret_cast<const void*>(indexer_plain_kernel<float>), 256, sizeof(float) * kPlainIndexerMaxElems},
  };
  for (const auto& k : ks) {
    const hipError_t e = check_launch_limits(k.fn, k.threads, k.dyn_lds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t check_indexer_kernels() {
  static PerDeviceCache cache;
  return once_per_device(cache, check_indexer_kernels_now);
}

hipError_t launch_indexer_candidates(const IndexerArgs& a, const IndexerCandidates& fo, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  const IndexerUnits un = indexer_units(a.n_q, a.ld);
  const int64_t n_units = un.n_kr * un.n_qb;
  if (n_units > (int64_t)1 << 30 || un.keys_per_unit % kIdxStageKeys != 0 || fo.n_kr != un.n_kr ||
      fo.row_cap != un.n_kr * un.keys_per_unit)
    return hipErrorInvalidValue;
  const int units_per_xcd = (int)((n_units + 7) / 8);
  return launch_kernel(indexer_lds_kernel<true>, dim3(units_per_xcd * 8), dim3(kIdx8Threads), 0, s, a.n_q, a.offset,
                       static_cast<const uint16_t*>(a.q_idx), a.w, static_cast<const uint16_t*>(a.k_idx),
                       static_cast<float*>(nullptr), a.ld, un.n_qb, (int)n_units, units_per_xcd, un.keys_per_unit, fo);
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (indexer_fast_path(a)) {
    switch (a.d_idx) {
      case 32: return launch_mfma<32>(a, s);
      case 64: return launch_mfma<64>(a, s);
      case 128: return launch_mfma<128>(a, s);
      case 256: return launch_mfma<256>(a, s);
    }
  }
  const int64_t gx = (a.ld + 255) / 256;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * (size_t)a.n_idx_heads * a.d_idx;
  if (a.bf16)
    return launch_kernel(indexer_plain_kernel<uint16_t>, dim3((unsigned)gx, a.n_q), dim3(256), lds, s, a.n_q,
                         a.offset, a.n_idx_heads, a.d_idx, static_cast<const uint16_t*>(a.q_idx), a.w,
                         static_cast<const uint16_t*>(a.k_idx), a.scores, a.ld);
  return launch_kernel(indexer_plain_kernel<float>, dim3((unsigned)gx, a.n_q), dim3(256), lds, s, a.n_q, a.offset,
                       a.n_idx_heads, a.d_idx, static_cast<const float*>(a.q_idx), a.w,
                       static_cast<const float*>(a.k_idx), a.scores, a.ld);
}

}  // namespace dsa
