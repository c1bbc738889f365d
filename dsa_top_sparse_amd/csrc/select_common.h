// select_common.h -- device code shared by the top-k selects (the select over
// a materialised score row, and the select over the candidates the fused
// indexer writes): block scans, histograms with bucket search, the threshold
// from a row's first keys, and the exact select and ordered emit over the
// candidates of a threshold (or over a whole row).
//
// Keys: the order-preserving uint32 image of a score (score_key), digits of
// 11 + 11 + 10 bits. The selected set is the top k in (score descending, key
// index ascending) order; indices are emitted ascending.
#pragma once

#include "common.h"

namespace dsa {

// Barrier for LDS traffic only: unlike __syncthreads() it leaves this
// thread's global loads in flight (the streaming passes prefetch across it).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the wave with DPP moves: shifts of 1, 2, 4 and 8
// lanes inside each row of 16, then row 0's total into row 1 and row 2's
// into row 3 (row_bcast:15), then the total of rows 0-1 into rows 2-3
// (row_bcast:31). Six dependent VALU steps instead of six LDS-crossbar
// shuffles.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xa, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xc, 0xf, false));
  return x;
}

// Adds this wave's OR / AND of the last 10 bits of `o` / `a` to the
// block's words *w_or / *w_and (one ballot per bit: no chain of dependent
// shuffles).
__device__ __forceinline__ void publish_low_bits_to(uint32_t* w_or, uint32_t* w_and, uint32_t o, uint32_t a) {
  uint32_t wo = 0u, wa = 0u;
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    wo |= (__ballot((o >> b) & 1u) != 0) ? (1u << b) : 0u;
    wa |= (__ballot(((a >> b) & 1u) == 0u) == 0) ? (1u << b) : 0u;
  }
  if ((threadIdx.x & 63) == 0) {
    atomicOr(w_or, wo);
    atomicAnd(w_and, wa);
  }
}

constexpr int kFsThreads = 256;
constexpr int kFsWaves = kFsThreads / kWave;
constexpr int kFsSlice = 4 * kFsThreads;  // keys per block-wide step (4 per thread)
constexpr int kFsGroup = 4;               // slices per compaction scan
constexpr int kFsGroupKeys = kFsGroup * kFsSlice;
constexpr int kFsBins = 2048;
constexpr int kFsCap = 4096;              // LDS candidate capacity
constexpr int kFsSample = 2048;           // keys of the threshold sample (the row's first)
constexpr int kFsSampleSlices = kFsSample / kFsSlice;
constexpr int kFsMaxRow = 65536;          // candidate indices are 16-bit
static_assert(kFsSampleSlices >= 1 && kFsSampleSlices <= kFsGroup, "sample inside the first group");

struct FsSmem {
  uint32_t hist[kFsBins / 2];  // 2048 bins of 16-bit counts, two to a word (counts of at most kFsCap keys)
  uint32_t ckey[kFsCap + 4];   // candidate keys (+ a spare entry); else a 2048-bin 32-bit histogram
  uint16_t cidx[kFsCap + 4];  // candidate key indices
  uint64_t scan[2][kFsWaves];
  uint32_t bc[4];
  uint32_t low_or, low_and;
};

__device__ __forceinline__ uint64_t fs_scan(uint64_t v, uint64_t* total, FsSmem& sm, int& buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t x = (static_cast<uint64_t>(wave_incl_scan(static_cast<uint32_t>(v >> 32))) << 32) |
                     wave_incl_scan(static_cast<uint32_t>(v));
  if (lane == kWave - 1) sm.scan[buf][wave] = x;
  lds_sync();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFsWaves; ++w) {
    const uint64_t t = sm.scan[buf][w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  buf ^= 1;
  *total = all;
  return before + x - v;
}

// Bucket of a 2048-bin histogram (top bin first) at which the running count
// reaches `need` (the histogram must hold at least `need`); its count and the
// count above it. PACKED: 16-bit counts, two to a word (bin b in word b / 2,
// the high half for odd b); else one 32-bit count a word. Every thread's bins
// are read before the scan's barrier, so the histogram may be overwritten
// once this returns.
template <bool PACKED>
__device__ __forceinline__ void fs_bucket(const uint32_t* hist, FsSmem& sm, uint32_t need, uint32_t* b_out,
                                          uint32_t* above_out, uint32_t* cnt_out, int& buf) {
  constexpr int per = kFsBins / kFsThreads;  // 8
  const int lo = threadIdx.x * per;
  uint32_t h[per];
  if (PACKED) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&hist[lo / 2]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[2 * e] = v[e] & 0xFFFFu;
      h[2 * e + 1] = v[e] >> 16;
    }
  } else {
#pragma unroll
    for (int q = 0; q < per; q += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&hist[lo + q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) h[q + e] = v[e];
    }
  }
  uint32_t local = 0;
#pragma unroll
  for (int b = 0; b < per; ++b) local += h[b];
  uint64_t total;
  const uint64_t excl = fs_scan(local, &total, sm, buf);
  const uint32_t above = static_cast<uint32_t>(total - excl - local);
  if (above < need && above + local >= need) {
    uint32_t run = above;
    bool found = false;
#pragma unroll
    for (int b = per - 1; b >= 0; --b) {
      if (!found && run + h[b] >= need) {
        sm.bc[0] = lo + b;
        sm.bc[1] = run;
        sm.bc[2] = h[b];
        found = true;
      }
      run += h[b];
    }
  }
  lds_sync();
  *b_out = sm.bc[0];
  *above_out = sm.bc[1];
  *cnt_out = sm.bc[2];
}

// One key into bin b of a histogram as fs_bucket reads it.
template <bool PACKED>
__device__ __forceinline__ void fs_count(uint32_t* hist, uint32_t b) {
  if (PACKED) atomicAdd(&hist[b >> 1], (b & 1u) ? 0x10000u : 1u);
  else atomicAdd(&hist[b], 1u);
}

// Zeroes a 2048-bin histogram (PACKED: 1024 words, else 2048).
template <bool PACKED>
__device__ __forceinline__ void fs_zero(uint32_t* a) {
  constexpr int words = PACKED ? kFsBins / 2 : kFsBins;
  for (int b = 4 * threadIdx.x; b < words; b += 4 * kFsThreads) *reinterpret_cast<u32x4*>(&a[b]) = u32x4{0u, 0u, 0u, 0u};
}

// The score whose order-preserving key is `key` (the inverse of score_key for
// keys of real scores); a key below that of -inf maps to -inf, so that every
// score compares >= it as its key does.
__device__ __forceinline__ float key_to_score(uint32_t key) {
  const float f = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
  return f != f ? -INFINITY : f;
}

// Elements base + 4 tid + e of the row (aligned 16-byte load, address clamped
// into the row: lanes past n read a valid element and are masked by the caller).
__device__ __forceinline__ f32x4 fs_load4(const float* __restrict__ row, int base, int n) {
  const int j = base + 4 * threadIdx.x;
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + min(j, (n - 1) & ~3)));
}

// Ordered compaction of one group of kFsGroup slices (keys base ..): every
// valid key >= lo goes to the candidate list at cbase + its rank; with
// with_hist the histogram of the written keys' top digit is built on the
// way. Returns the group's count (also of keys past the capacity, which are
// not written).
__device__ __forceinline__ uint32_t fs_compact(FsSmem& sm, int& buf, const uint32_t (&key)[kFsGroup][4], int base,
                                               int n, uint32_t lo, uint32_t cbase, bool with_hist) {
  const int tid = threadIdx.x;
  uint64_t packed = 0;  // kFsGroup x 16-bit per-slice counts (a slice holds <= 1024 keys)
#pragma unroll
  for (int s = 0; s < kFsGroup; ++s) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += (base + s * kFsSlice + 4 * tid + e < n) && key[s][e] >= lo;
    packed |= static_cast<uint64_t>(c) << (16 * s);
  }
  uint64_t tot;
  const uint64_t excl = fs_scan(packed, &tot, sm, buf);
  uint32_t slice_base = cbase;
#pragma unroll
  for (int s = 0; s < kFsGroup; ++s) {
    uint32_t pos = slice_base + static_cast<uint32_t>((excl >> (16 * s)) & 0xFFFF);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = base + s * kFsSlice + 4 * tid + e;
      if (j < n && key[s][e] >= lo) {
        if (pos < static_cast<uint32_t>(kFsCap)) {
          sm.ckey[pos] = key[s][e];
          sm.cidx[pos] = static_cast<uint16_t>(j);
          if (with_hist) fs_count<true>(sm.hist, key[s][e] >> 21);
        }
        ++pos;
      }
    }
    slice_base += static_cast<uint32_t>((tot >> (16 * s)) & 0xFFFF);
  }
  return slice_base - cbase;
}

// Refine and emit. On entry the keys with (key >> shift) == prefix hold the
// k-th largest key; `need` of them are still to be kept and `tie_cnt` exist
// (shift 21: prefix is the top digit; 10: the top 22 bits). With low_known,
// sm.low_or / sm.low_and hold the OR / AND of the last 10 bits over a superset
// of those keys. With in_lds the n_cand candidates (every key at or above the
// k-th, maybe more) sit in LDS in index order; otherwise every step streams
// the row from global memory.
__device__ __forceinline__ void fs_tail(FsSmem& sm, int& buf, const float* __restrict__ row, int n, int k,
                                        int32_t* __restrict__ out, uint32_t prefix, int shift, uint32_t need,
                                        uint32_t tie_cnt, bool low_known, bool in_lds, int n_cand) {
  const int tid = threadIdx.x;
  while (shift > 0 && tie_cnt != need) {
    if (shift == 10 && low_known && ((sm.low_or ^ sm.low_and) & 1023u) == 0u) {
      prefix = (prefix << 10) | (sm.low_or & 1023u);  // the one key value left
      shift = 0;
      break;
    }
    const bool first = shift == 21;
    const int nshift = first ? 10 : 0;
    const uint32_t dmask = first ? 2047u : 1023u;
    // candidates (at most kFsCap): the packed histogram; a streamed row: 32-bit
    // counts in the candidate area, which is then unused
    if (in_lds) fs_zero<true>(sm.hist);
    else fs_zero<false>(sm.ckey);
    __syncthreads();
    uint32_t lo = 0u, la = 0xFFFFFFFFu;
    if (in_lds) {
      for (int c = 4 * tid; c < n_cand; c += 4 * kFsThreads) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(&sm.ckey[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + e < n_cand && (kv[e] >> shift) == prefix) {
            fs_count<true>(sm.hist, (kv[e] >> nshift) & dmask);
            lo |= kv[e];
            la &= kv[e];
          }
        }
      }
    } else {
      for (int base = 0; base < n; base += kFsSlice) {
        const f32x4 v = fs_load4(row, base, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = score_key(v[e]);
          if (base + 4 * tid + e < n && (key >> shift) == prefix) {
            fs_count<false>(sm.ckey, (key >> nshift) & dmask);
            lo |= key;
            la &= key;
          }
        }
      }
    }
    const bool publish = first && !low_known;
    if (publish) publish_low_bits_to(&sm.low_or, &sm.low_and, lo, la);
    __syncthreads();
    uint32_t b, above, cnt;
    if (in_lds) fs_bucket<true>(sm.hist, sm, need, &b, &above, &cnt, buf);
    else fs_bucket<false>(sm.ckey, sm, need, &b, &above, &cnt, buf);
    need -= above;
    prefix = (prefix << (shift - nshift)) | b;
    shift = nshift;
    tie_cnt = cnt;
    low_known = low_known || publish;
  }
  const uint32_t r = need;  // keys with (key >> shift) == prefix to keep, lowest indices first

  uint32_t gt_base = 0, tie_base = 0;
  if (in_lds) {
    // Two slices per scan: each 32-bit half packs the two slices' counts in 16-bit fields.
    for (int base = 0; base < n_cand; base += 2 * kFsSlice) {
      uint32_t gt[2][4], tie[2][4];
      int32_t jj[2][4];
      uint32_t cgt = 0, ctie = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c0 = base + h * kFsSlice + 4 * tid;
        u32x4 kv = {0u, 0u, 0u, 0u};
        uint16_t ix[4] = {0, 0, 0, 0};
        if (c0 < n_cand) {
          kv = *reinterpret_cast<const u32x4*>(&sm.ckey[c0]);
          const u32x2 p = *reinterpret_cast<const u32x2*>(&sm.cidx[c0]);
          ix[0] = p[0] & 0xFFFF;
          ix[1] = p[0] >> 16;
          ix[2] = p[1] & 0xFFFF;
          ix[3] = p[1] >> 16;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool valid = c0 + e < n_cand;
          jj[h][e] = ix[e];
          gt[h][e] = valid && (kv[e] >> shift) > prefix;
          tie[h][e] = valid && (kv[e] >> shift) == prefix;
          cgt += gt[h][e] << (16 * h);
          ctie += tie[h][e] << (16 * h);
        }
      }
      uint64_t tot;
      const uint64_t excl = fs_scan((static_cast<uint64_t>(ctie) << 32) | cgt, &tot, sm, buf);
      const uint32_t egt = static_cast<uint32_t>(excl), etie = static_cast<uint32_t>(excl >> 32);
      const uint32_t tgt = static_cast<uint32_t>(tot), ttie = static_cast<uint32_t>(tot >> 32);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t g = gt_base + (h ? (tgt & 0xFFFFu) + (egt >> 16) : (egt & 0xFFFFu));
        uint32_t t = tie_base + (h ? (ttie & 0xFFFFu) + (etie >> 16) : (etie & 0xFFFFu));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t pos = gt[h][e] ? g + min(t, r) : g + t;  // < k by construction
          if ((gt[h][e] || (tie[h][e] && t < r)) && pos < static_cast<uint32_t>(k)) out[pos] = jj[h][e];
          g += gt[h][e];
          t += tie[h][e];
        }
      }
      gt_base += (tgt & 0xFFFFu) + (tgt >> 16);
      tie_base += (ttie & 0xFFFFu) + (ttie >> 16);
    }
  } else {
    for (int base = 0; base < n; base += kFsSlice) {
      const f32x4 v = fs_load4(row, base, n);
      uint32_t gt[4], tie[4];
      uint32_t cgt = 0, ctie = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = base + 4 * tid + e < n;
        const uint32_t key = score_key(v[e]);
        gt[e] = valid && (key >> shift) > prefix;
        tie[e] = valid && (key >> shift) == prefix;
        cgt += gt[e];
        ctie += tie[e];
      }
      uint64_t tot;
      const uint64_t excl = fs_scan((static_cast<uint64_t>(ctie) << 32) | cgt, &tot, sm, buf);
      uint32_t g = gt_base + static_cast<uint32_t>(excl);
      uint32_t t = tie_base + static_cast<uint32_t>(excl >> 32);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = base + 4 * tid + e;
        const uint32_t pos = gt[e] ? g + min(t, r) : g + t;
        if ((gt[e] || (tie[e] && t < r)) && pos < static_cast<uint32_t>(k)) out[pos] = j;
        g += gt[e];
        t += tie[e];
      }
      gt_base += static_cast<uint32_t>(tot);
      tie_base += static_cast<uint32_t>(tot >> 32);
    }
  }
}

// Threshold from a row's first S = min(n, kFsSample) keys, held in cur[s]
// (s < kFsSampleSlices; elements s * kFsSlice + 4 tid + e): their key of
// rank rs, a fifth above the rank the k-th key is expected at (plus 16), to
// 22 bits. Expects sm.hist (packed) and the first kFsBins words of sm.ckey
// zeroed before a barrier; returns with sm.hist zeroed again and sm.ckey
// free.
__device__ __forceinline__ uint32_t fs_sample_tau(FsSmem& sm, int& buf, const f32x4* cur, int n, int k) {
  const int tid = threadIdx.x;
  const int S = min(n, kFsSample);
  const uint32_t rs = static_cast<uint32_t>(
      min<int64_t>(S, (static_cast<int64_t>(k) * S * 6 + 5 * static_cast<int64_t>(n) - 1) /
                              (5 * static_cast<int64_t>(n)) + 16));
  uint32_t skey[kFsSampleSlices][4];
#pragma unroll
  for (int s = 0; s < kFsSampleSlices; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      skey[s][e] = score_key(cur[s][e]);
      if (s * kFsSlice + 4 * tid + e < S) fs_count<true>(sm.hist, skey[s][e] >> 21);
    }
  lds_sync();
  uint32_t bs, above_s, cnt_s;
  fs_bucket<true>(sm.hist, sm, rs, &bs, &above_s, &cnt_s, buf);
#pragma unroll
  for (int s = 0; s < kFsSampleSlices; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (s * kFsSlice + 4 * tid + e < S && (skey[s][e] >> 21) == bs)
        fs_count<false>(sm.ckey, (skey[s][e] >> 10) & 2047u);
  fs_zero<true>(sm.hist);  // read by fs_bucket above before its scan: free again
  lds_sync();
  uint32_t b2, above_2, cnt_2;
  fs_bucket<false>(sm.ckey, sm, rs - above_s, &b2, &above_2, &cnt_2, buf);
  return (bs << 21) | (b2 << 10);
}

// The exact select and the ordered emit over nc candidates in LDS: raw score
// bits in sm.ckey, key indices in sm.cidx, in index order, holding every key
// >= tau (tau's last 10 bits zero), with k <= nc <= kFsCap. Expects sm.hist
// zeroed and sm.low_or / sm.low_and reset (0 / 0x3FF) before a barrier.
__device__ __forceinline__ void fs_select_candidates(FsSmem& sm, int& buf, const float* __restrict__ row, int n,
                                                     int k, int32_t* __restrict__ out, uint32_t tau, int nc) {
  const int tid = threadIdx.x;
  // Candidate scores to keys, the histogram of their top 22 bits relative to
  // tau's (the last bin collects everything 2,047 steps above), and the OR /
  // AND of the last 10 bits of the keys below that last bin.
  const uint32_t tau22 = tau >> 10;
  uint32_t lo = 0u, la = 0xFFFFFFFFu;
  for (int c = 4 * tid; c < nc; c += 4 * kFsThreads) {
    u32x4 kv = *reinterpret_cast<const u32x4*>(&sm.ckey[c]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[e] = score_key(__uint_as_float(kv[e]));
      const uint32_t d = (kv[e] >> 10) - tau22;
      if (c + e < nc) {
        fs_count<true>(sm.hist, min(d, 2047u));
        if (d < 2047u) {
          lo |= kv[e];
          la &= kv[e];
        }
      }
    }
    *reinterpret_cast<u32x4*>(&sm.ckey[c]) = kv;
  }
  publish_low_bits_to(&sm.low_or, &sm.low_and, lo, la);
  __syncthreads();
  uint32_t b, above, cnt;
  fs_bucket<true>(sm.hist, sm, static_cast<uint32_t>(k), &b, &above, &cnt, buf);
  if (b < 2047u) {  // the k-th key's top 22 bits are tau22 + b
    fs_tail(sm, buf, row, n, k, out, tau22 + b, 10, static_cast<uint32_t>(k) - above, cnt, true, true, nc);
    return;
  }
  // the k-th key lies 2,047 or more steps above tau: the top digit from the candidates
  fs_zero<true>(sm.hist);
  if (tid == 0) {
    sm.low_or = 0u;
    sm.low_and = 0x3FFu;
  }
  __syncthreads();
  for (int c = 4 * tid; c < nc; c += 4 * kFsThreads) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(&sm.ckey[c]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < nc) fs_count<true>(sm.hist, kv[e] >> 21);
  }
  __syncthreads();
  fs_bucket<true>(sm.hist, sm, static_cast<uint32_t>(k), &b, &above, &cnt, buf);
  fs_tail(sm, buf, row, n, k, out, b, 21, static_cast<uint32_t>(k) - above, cnt, false, true, nc);
}

// The select of a whole row of n > k scores in global memory (16-byte
// aligned), with no threshold: the exact top digit from a full histogram pass
// (32-bit counts, in the candidate area), then the keys at or above it
// compacted into LDS if they fit, else every later step streams the row.
// Expects a barrier before (LDS free).
__device__ __forceinline__ void fs_select_row(FsSmem& sm, int& buf, const float* __restrict__ row, int n, int k,
                                              int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  fs_zero<false>(sm.ckey);
  if (tid == 0) {
    sm.low_or = 0u;
    sm.low_and = 0x3FFu;
  }
  __syncthreads();
  for (int base = 0; base < n; base += kFsSlice) {
    const f32x4 v = fs_load4(row, base, n);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (base + 4 * tid + e < n) fs_count<false>(sm.ckey, score_key(v[e]) >> 21);
  }
  __syncthreads();
  uint32_t b1, above1, cnt1;
  fs_bucket<false>(sm.ckey, sm, static_cast<uint32_t>(k), &b1, &above1, &cnt1, buf);
  const bool fits = above1 + cnt1 <= static_cast<uint32_t>(kFsCap);
  if (fits) {
    uint32_t cbase = 0;
    for (int base = 0; base < n; base += kFsGroupKeys) {
      uint32_t key[kFsGroup][4];
#pragma unroll
      for (int s = 0; s < kFsGroup; ++s) {
        const f32x4 v = fs_load4(row, base + s * kFsSlice, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[s][e] = score_key(v[e]);
      }
      cbase += fs_compact(sm, buf, key, base, n, b1 << 21, cbase, false);
    }
    __syncthreads();
  }
  fs_tail(sm, buf, row, n, k, out, b1, 21, static_cast<uint32_t>(k) - above1, cnt1, false, fits,
          static_cast<int>(above1 + cnt1));
}

}  // namespace dsa
