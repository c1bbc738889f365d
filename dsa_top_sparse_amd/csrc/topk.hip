// topk.hip -- step 2 of the DSA prefill path: per-query top-k selection.
//
// For query i (absolute position p = offset + i) the causal scores are
// scores[i][0 .. p]. If p + 1 <= k every causal key is kept; otherwise the k
// keys first in (score descending, key index ascending) order are kept. The
// kept indices are written ascending, padded with -1 to k. (feedman.me page,
// the paragraph on the work that is not a matmul: each query gathers its top
// 2,048 keys; the tie rule is this library's contract: a tie at the
// threshold goes to the lower key index.)
//
// One workgroup per query row, an exact radix select on the order-preserving
// uint32 image ("key") of each score, with digits of 11 + 11 + 10 bits (the
// streamed kernel for long rows: 12 + 10 + 10). Two kernels:
//
// topk_filter_kernel (rows of at most 65,536 keys, 16-byte aligned rows; the
// hot path): five rows share a CU (about 29 KB of LDS each).
//   sample   : the histogram of the row's first 2,048 keys, two levels deep,
//              gives tau, the sample's key of rank a fifth above where the
//              k-th key is expected (plus 16), to 22 bits;
//   stream   : one pass over the row keeps every key >= tau (a float compare
//              against the score whose key is tau), in index order, in LDS;
//   select   : over those candidates only: a histogram of their top 22 bits
//              relative to tau's gives the k-th key's top 22 bits; when the
//              last 10 bits agree over the candidates near tau (as they do
//              for integer-valued scores) that is the exact threshold T, else
//              one more 10-bit level over the candidates finds it;
//   emit     : in index order, keep key > T, and key == T while fewer than r
//              ties have been kept (r = how many of the keys equal to T fit);
//              the output position of a kept key is (#greater before it) +
//              min(#ties before it, r), from packed block scans.
//   If the sample misleads (fewer than k keys >= tau, or more than fit in
//   LDS), the row is selected again without it: a full histogram pass, then
//   the keys at or above the k-th key's top digit are compacted (if they fit;
//   otherwise every later step streams the row from global memory).
//
// topk_kernel (longer or unaligned rows): the 12-bit histogram of the row's
// first 8,192 keys gives a speculative bucket bs a margin below the k-th
// key's expected place; one streamed pass builds the full histogram while it
// compacts every key with top bits >= bs; if the exact bucket b1 is >= bs and
// those keys fit in LDS the row has been read once, else a second pass
// compacts the keys >= b1; if they do not fit either, the refine and emit
// passes re-read the row.
//
// The result is the same on every path. Block scans run their wave part on
// DPP row shifts and broadcasts.
#include <type_traits>

#include "common.h"
#include "select_common.h"
#include "device_checks.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kSlice = 4 * kTkThreads;  // elements per block-wide step (4 per thread)
constexpr int kBins1 = 4096;            // top 12 bits
constexpr int kBins2 = 1024;            // 10 bits
constexpr int kTkCap = 6144;            // LDS candidate capacity

struct TopkSmem {
  uint32_t hist[kBins1];
  u32x2 cand[kTkCap];  // (key, index) in index order
  uint64_t scan[2][kTkWaves];
  uint32_t bc[4];
  uint32_t low_or, low_and;  // OR / AND of the boundary bucket's keys (last 10 bits)
};

// Block-wide exclusive scan of a uint64 (callers pack independent counters in
// bit fields that cannot overflow into each other). `buf` alternates between
// calls so that a single barrier per scan suffices.
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t* total, TopkSmem& sm, int& buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // The two 32-bit halves scan separately: no field carries across them.
  const uint64_t x = (static_cast<uint64_t>(wave_incl_scan(static_cast<uint32_t>(v >> 32))) << 32) |
                     wave_incl_scan(static_cast<uint32_t>(v));
  if (lane == kWave - 1) sm.scan[buf][wave] = x;
  lds_sync();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint64_t t = sm.scan[buf][w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  buf ^= 1;
  *total = all;
  return before + x - v;
}

// Finds the bucket b (scanning from the top bin down) at which the running
// count of keys reaches `need`; returns b and the count strictly above it.
// Requires that the histogram holds at least `need` keys.
__device__ __forceinline__ void select_bucket(const uint32_t* hist, TopkSmem& sm, int nbins, uint32_t need,
                                              uint32_t* b_out,
                                              uint32_t* above_out, uint32_t* cnt_out, int& buf) {
  const int per = nbins / kTkThreads;
  const int lo = threadIdx.x * per;
  uint32_t local = 0;
  for (int b = 0; b < per; ++b) local += hist[lo + b];
  uint64_t total;
  const uint64_t excl = block_excl_scan(local, &total, sm, buf);
  const uint32_t above = static_cast<uint32_t>(total - excl - local);  // keys in higher bins
  if (above < need && above + local >= need) {
    uint32_t run = above;
    for (int b = lo + per - 1; b >= lo; --b) {
      const uint32_t h = hist[b];
      if (run + h >= need) {
        sm.bc[0] = b;
        sm.bc[1] = run;
        sm.bc[2] = h;
        break;
      }
      run += h;
    }
  }
  lds_sync();  // LDS only: loads of the streaming select stay in flight
  *b_out = sm.bc[0];
  *above_out = sm.bc[1];
  *cnt_out = sm.bc[2];
}

__device__ __forceinline__ void publish_low_bits(TopkSmem& sm, uint32_t o, uint32_t a) {
  publish_low_bits_to(&sm.low_or, &sm.low_and, o, a);
}

// Loads elements base + 4*tid + e (e < 4) of the row. Elements past n hold
// unspecified values: every user tests e < n itself. The aligned load is not
// predicated (its address is clamped into the row), so the compiler can wait
// for each load separately instead of for all loads in flight.
template <bool ALIGNED>
__device__ __forceinline__ f32x4 load4(const float* __restrict__ row, int base, int n) {
  const int j = base + 4 * threadIdx.x;
  f32x4 v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (ALIGNED) {
    v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + min(j, (n - 1) & ~3)));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e < n) v[e] = row[j + e];
  }
  return v;
}

// Refine and emit, after bucket b1 (holding the k-th largest key; above1 keys
// lie in higher buckets, cnt1 in b1) is known and, when in_lds, the keys with
// top bits >= b1 sit in LDS in index order.
template <bool ALIGNED>
__device__ __forceinline__ void select_tail(TopkSmem& sm, int& buf, const float* __restrict__ row, int n, int k,
                                            int32_t* __restrict__ out, uint32_t b1, uint32_t above1, uint32_t cnt1,
                                            bool in_lds, int n_cand) {
  const int tid = threadIdx.x;

  // ---- refine: exact threshold inside bucket b1 with two 10-bit digits.
  uint32_t need = static_cast<uint32_t>(k) - above1;
  uint32_t prefix = b1;  // decided top bits, right-aligned
  int shift = 20;        // number of undecided low bits
  uint32_t tie_cnt = cnt1;
  for (int level = 0; level < 2 && tie_cnt != need; ++level) {
    const int nshift = shift - 10;
    for (int b = tid; b < kBins2; b += kTkThreads) sm.hist[b] = 0;
    __syncthreads();
    // The first level also gathers the OR and the AND of the bucket's keys:
    // where their last 10 bits agree over the whole bucket, the keys left
    // after this level are all equal and the second level is not needed.
    uint32_t lo = 0u, la = 0xFFFFFFFFu;
    if (in_lds) {
      for (int c = tid; c < n_cand; c += kTkThreads) {
        const uint32_t key = sm.cand[c][0];
        if ((key >> shift) == prefix) {
          atomicAdd(&sm.hist[(key >> nshift) & 1023u], 1u);
          lo |= key;
          la &= key;
        }
      }
    } else {
      for (int base = 0; base < n; base += kSlice) {
        const f32x4 v = load4<ALIGNED>(row, base, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = score_key(v[e]);
          if (base + 4 * tid + e < n && (key >> shift) == prefix) {
            atomicAdd(&sm.hist[(key >> nshift) & 1023u], 1u);
            lo |= key;
            la &= key;
          }
        }
      }
    }
    if (level == 0) publish_low_bits(sm, lo, la);
    __syncthreads();
    uint32_t b, above, cnt;
    select_bucket(sm.hist, sm, kBins2, need, &b, &above, &cnt, buf);
    need -= above;
    prefix = (prefix << 10) | b;
    shift = nshift;
    tie_cnt = cnt;
    if (level == 0 && tie_cnt != need && ((sm.low_or ^ sm.low_and) & 1023u) == 0u) {
      prefix = (prefix << 10) | (sm.low_or & 1023u);  // the single key value left
      shift = 0;
      break;
    }
  }
  // Keys with (key >> shift) > prefix are kept; of those equal, the first `need`.
  const uint32_t r = need;

  // ---- emit in index order.
  uint32_t gt_base = 0, tie_base = 0;
  if (in_lds) {
    // Two slices per block scan: each 32-bit half of the scanned value packs
    // the two slices' counts in 16-bit fields (a slice holds <= 2048 keys).
    for (int base = 0; base < n_cand; base += 2 * kSlice) {
      uint32_t gt[2][4], tie[2][4];
      int32_t jj[2][4];
      uint32_t cgt = 0, ctie = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = base + h * kSlice + 4 * tid + e;
          const bool valid = c < n_cand;
          const u32x2 kv = valid ? sm.cand[c] : u32x2{0u, 0xFFFFFFFFu};
          const uint32_t key = kv[0];
          jj[h][e] = static_cast<int32_t>(kv[1]);
          gt[h][e] = valid && (key >> shift) > prefix;
          tie[h][e] = valid && (key >> shift) == prefix;
          cgt += gt[h][e] << (16 * h);
          ctie += tie[h][e] << (16 * h);
        }
      }
      uint64_t tot;
      const uint64_t excl = block_excl_scan((static_cast<uint64_t>(ctie) << 32) | cgt, &tot, sm, buf);
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
    for (int base = 0; base < n; base += kSlice) {
      const f32x4 v = load4<ALIGNED>(row, base, n);
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
      const uint64_t excl = block_excl_scan((static_cast<uint64_t>(ctie) << 32) | cgt, &tot, sm, buf);
      uint32_t g = gt_base + static_cast<uint32_t>(excl);
      uint32_t t = tie_base + static_cast<uint32_t>(excl >> 32);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = base + 4 * tid + e;
        const uint32_t pos = gt[e] ? g + min(t, r) : g + t;  // < k by construction
        if ((gt[e] || (tie[e] && t < r)) && pos < static_cast<uint32_t>(k)) out[pos] = j;
        g += gt[e];
        t += tie[e];
      }
      gt_base += static_cast<uint32_t>(tot);
      tie_base += static_cast<uint32_t>(tot >> 32);
    }
  }
}

template <bool ALIGNED>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(int offset, int k, const float* __restrict__ scores,
                                                          int64_t ld, int32_t* __restrict__ idx) {
  lds_poison();
  __shared__ TopkSmem sm;
  int buf = 0;
  const int i = blockIdx.x;
  const int n = offset + i + 1;  // causal keys 0 .. p (fits int32: validated on the host)
  int32_t* __restrict__ out = idx + static_cast<int64_t>(i) * k;
  if (n <= k) {
    for (int t = threadIdx.x; t < k; t += kTkThreads) out[t] = t < n ? t : -1;
    return;
  }
  const float* __restrict__ row = scores + static_cast<int64_t>(i) * ld;
  const int tid = threadIdx.x;

  // ---- histogram of group 0 (keys 0 .. 8,191), which stays in registers.
  for (int b = 4 * tid; b < kBins1; b += 4 * kTkThreads) *reinterpret_cast<u32x4*>(&sm.hist[b]) = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) {
    sm.low_or = 0u;
    sm.low_and = 0xFFFFFu;
  }
  __syncthreads();
  f32x4 v[4], nx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) v[s] = load4<ALIGNED>(row, s * kSlice, n);
#pragma unroll
  for (int s = 0; s < 4; ++s) nx[s] = load4<ALIGNED>(row, 4 * kSlice + s * kSlice, n);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (s * kSlice + 4 * tid + e < n) atomicAdd(&sm.hist[score_key(v[s][e]) >> 20], 1u);
  lds_sync();  // the loads of group 1 stay in flight

  // ---- speculative candidate bucket bs: where group 0 reaches a rank a
  // quarter above the k-th key's expected rank in it. If the exact bucket b1
  // found below is >= bs and the keys with top bits >= bs fit in LDS, the one
  // pass below has already compacted every key the select needs (and some
  // more, which the refine and emit steps pass over); else the row is read
  // a second time, as in the plain two-pass select.
  const int n0 = min(n, 4 * kSlice);
  uint32_t need_s = static_cast<uint32_t>((static_cast<int64_t>(k) * n0 + n - 1) / n);
  need_s += need_s / 4 + 64;
  const bool spec = n > 4 * kSlice && need_s <= static_cast<uint32_t>(n0);
  uint32_t bs = 0;
  if (spec) {
    uint32_t a_s, c_s;
    select_bucket(sm.hist, sm, kBins1, need_s, &bs, &a_s, &c_s, buf);
  }

  // ---- one pass: the histogram of groups 1.. and, when speculating, the
  // ordered compaction of every key with top bits >= bs. The loads of the
  // group after next go out before this group is counted.
  uint32_t cbase = 0;
  for (int base = 0; base < n; base += 4 * kSlice) {
    f32x4 nn[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) nn[s] = load4<ALIGNED>(row, base + 8 * kSlice + s * kSlice, n);
    uint32_t key[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) key[s][e] = score_key(v[s][e]);
    if (base > 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (base + s * kSlice + 4 * tid + e < n) atomicAdd(&sm.hist[key[s][e] >> 20], 1u);
    }
    if (spec) {
      uint64_t packed = 0;  // 4 x 16-bit per-slice counts (each slice total <= 2048)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c += (base + s * kSlice + 4 * tid + e < n) && (key[s][e] >> 20) >= bs;
        packed |= static_cast<uint64_t>(c) << (16 * s);
      }
      uint64_t tot;
      const uint64_t excl = block_excl_scan(packed, &tot, sm, buf);
      uint32_t slice_base = cbase;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t pos = slice_base + static_cast<uint32_t>((excl >> (16 * s)) & 0xFFFF);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = base + s * kSlice + 4 * tid + e;
          if (j < n && (key[s][e] >> 20) >= bs && pos < static_cast<uint32_t>(kTkCap)) {
            sm.cand[pos] = u32x2{key[s][e], static_cast<uint32_t>(j)};
            ++pos;
          }
        }
        slice_base += static_cast<uint32_t>((tot >> (16 * s)) & 0xFFFF);
      }
      cbase = slice_base;  // every key >= bs so far, also those past the capacity
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v[s] = nx[s];
      nx[s] = nn[s];
    }
  }
  __syncthreads();
  uint32_t b1, above1, cnt1;
  select_bucket(sm.hist, sm, kBins1, static_cast<uint32_t>(k), &b1, &above1, &cnt1, buf);
  const bool spec_ok = spec && b1 >= bs && cbase <= static_cast<uint32_t>(kTkCap);
  const bool in_lds = spec_ok || above1 + cnt1 <= static_cast<uint32_t>(kTkCap);
  int n_cand = static_cast<int>(spec_ok ? cbase : above1 + cnt1);

  // ---- second read (speculation missed): ordered compaction of every key
  // with top bits >= b1 into LDS.
  if (in_lds && !spec_ok) {
    cbase = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = load4<ALIGNED>(row, s * kSlice, n);
    for (int base = 0; base < n; base += 4 * kSlice) {
#pragma unroll
      for (int s = 0; s < 4; ++s) nx[s] = load4<ALIGNED>(row, base + 4 * kSlice + s * kSlice, n);
      uint32_t key[4][4];
      uint64_t packed = 0;  // 4 x 16-bit per-slice counts (each slice total <= 2048)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          key[s][e] = score_key(v[s][e]);
          const bool f = (base + s * kSlice + 4 * tid + e < n) && (key[s][e] >> 20) >= b1;
          c += f;
        }
        packed |= static_cast<uint64_t>(c) << (16 * s);
      }
      uint64_t tot;
      const uint64_t excl = block_excl_scan(packed, &tot, sm, buf);
      uint32_t slice_base = cbase;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t pos = slice_base + static_cast<uint32_t>((excl >> (16 * s)) & 0xFFFF);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = base + s * kSlice + 4 * tid + e;
          if (j < n && (key[s][e] >> 20) >= b1 && pos < static_cast<uint32_t>(kTkCap)) {
            sm.cand[pos] = u32x2{key[s][e], static_cast<uint32_t>(j)};
            ++pos;
          }
        }
        slice_base += static_cast<uint32_t>((tot >> (16 * s)) & 0xFFFF);
      }
      cbase = slice_base;
#pragma unroll
      for (int s = 0; s < 4; ++s) v[s] = nx[s];
    }
  }
  __syncthreads();
  select_tail<ALIGNED>(sm, buf, row, n, k, out, b1, above1, cnt1, in_lds, n_cand);
}

// The filtered select over a materialised score row (rows of at most
// kFsMaxRow keys, 16-byte aligned): the threshold from the row's first keys,
// one streamed pass that keeps every key >= it, then the select over those
// candidates; a row the sample misleads is selected again without it.
__global__ __launch_bounds__(kFsThreads) void topk_filter_kernel(int offset, int k, const float* __restrict__ scores,
                                                                 int64_t ld, int32_t* __restrict__ idx) {
  lds_poison();
  __shared__ FsSmem sm;
  int buf = 0;
  const int i = blockIdx.x;
  const int n = offset + i + 1;  // <= kFsMaxRow: checked on the host
  int32_t* __restrict__ out = idx + static_cast<int64_t>(i) * k;
  if (n <= k) {
    for (int t = threadIdx.x; t < k; t += kFsThreads) out[t] = t < n ? t : -1;
    return;
  }
  const float* __restrict__ row = scores + static_cast<int64_t>(i) * ld;
  const int tid = threadIdx.x;

  // The first two groups go out at once; the sample is the start of group 0.
  f32x4 cur[kFsGroup], nxt[kFsGroup];
#pragma unroll
  for (int s = 0; s < kFsGroup; ++s) cur[s] = fs_load4(row, s * kFsSlice, n);
#pragma unroll
  for (int s = 0; s < kFsGroup; ++s) nxt[s] = fs_load4(row, kFsGroupKeys + s * kFsSlice, n);
  fs_zero<true>(sm.hist);
  fs_zero<false>(sm.ckey);  // the sample's second-level histogram
  if (tid == 0) {
    sm.low_or = 0u;  // OR / AND of the last 10 bits of the keys near the threshold
    sm.low_and = 0x3FFu;
  }
  lds_sync();
  const uint32_t tau = fs_sample_tau(sm, buf, cur, n, k);

  // ---- one streamed pass: every key >= tau, in index order, into LDS as the
  // raw score bits. The test is a float compare against tf, the score whose
  // key is tau (same order, -0 equal to +0), and only the last group needs
  // the row-end mask. Loads run two groups ahead.
  const float tf = key_to_score(tau);
  uint32_t cbase = 0;
  // One group: flags, their block scan, the ordered writes. FULL groups lie
  // inside the row and skip the row-end mask.
  auto process = [&](const f32x4(&g)[kFsGroup], int base, auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    const int j0 = base + 4 * tid;
    uint32_t f[kFsGroup][4];  // 1 = candidate
    uint64_t packed = 0;      // kFsGroup x 16-bit per-slice counts (a slice holds <= 1024 keys)
#pragma unroll
    for (int s = 0; s < kFsGroup; ++s) {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[s][e] = (g[s][e] >= tf && (FULL || j0 + s * kFsSlice + e < n)) ? 1u : 0u;
      packed |= static_cast<uint64_t>(f[s][0] + f[s][1] + f[s][2] + f[s][3]) << (16 * s);
    }
    uint64_t tot;
    const uint64_t excl = fs_scan(packed, &tot, sm, buf);
#pragma unroll
    for (int s = 0; s < kFsGroup; ++s) {
      // positions past the capacity (the row then takes the fallback) all go
      // to the spare entry at kFsCap
      uint32_t pos = cbase + static_cast<uint32_t>((excl >> (16 * s)) & 0xFFFF);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (f[s][e]) {
          const uint32_t q = min(pos, static_cast<uint32_t>(kFsCap));
          sm.ckey[q] = __float_as_uint(g[s][e]);
          sm.cidx[q] = static_cast<uint16_t>(j0 + s * kFsSlice + e);
        }
        pos += f[s][e];
      }
      cbase += static_cast<uint32_t>((tot >> (16 * s)) & 0xFFFF);
    }
  };
  // Three register sets in turn (no copies between them): while one group is
  // processed, the next two are in flight.
  f32x4 third[kFsGroup];
#pragma unroll
  for (int s = 0; s < kFsGroup; ++s) third[s] = fs_load4(row, 2 * kFsGroupKeys + s * kFsSlice, n);
  auto step = [&](f32x4(&g)[kFsGroup], int base) {
    if (base + kFsGroupKeys <= n) process(g, base, std::true_type{});
    else process(g, base, std::false_type{});
#pragma unroll
    for (int s = 0; s < kFsGroup; ++s) g[s] = fs_load4(row, base + 3 * kFsGroupKeys + s * kFsSlice, n);
  };
  for (int base = 0; base < n; base += 3 * kFsGroupKeys) {
    step(cur, base);
    if (base + kFsGroupKeys >= n) break;
    step(nxt, base + kFsGroupKeys);
    if (base + 2 * kFsGroupKeys >= n) break;
    step(third, base + 2 * kFsGroupKeys);
  }
  lds_sync();

  if (cbase >= static_cast<uint32_t>(k) && cbase <= static_cast<uint32_t>(kFsCap)) {
    fs_select_candidates(sm, buf, row, n, k, out, tau, static_cast<int>(cbase));
    return;
  }
  fs_select_row(sm, buf, row, n, k, out);
}

hipError_t check_topk_kernels_now() {
  const void* ks[] = {reinterpret_cast<const void*>(topk_kernel<true>), reinterpret_cast<const void*>(topk_kernel<false>)};
  for (const void* k : ks) {
    const hipError_t e = check_launch_limits(k, kTkThreads, 0);
    if (e != hipSuccess) return e;
  }
  return check_launch_limits(reinterpret_cast<const void*>(topk_filter_kernel), kFsThreads, 0);
}

}  // namespace

hipError_t check_topk_kernels() {
  static PerDeviceCache cache;
  return once_per_device(cache, check_topk_kernels_now);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  const bool aligned = (a.ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.scores) & 15) == 0);
  const int64_t n_max = (int64_t)a.offset + a.n_q;  // longest causal row
  const dim3 grid(a.n_q), block(kTkThreads);
  if (aligned && n_max <= kFsMaxRow)
    return launch_kernel(topk_filter_kernel, grid, dim3(kFsThreads), 0, s, a.offset, a.top_k, a.scores, a.ld, a.idx);
  if (aligned) return launch_kernel(topk_kernel<true>, grid, block, 0, s, a.offset, a.top_k, a.scores, a.ld, a.idx);
  return launch_kernel(topk_kernel<false>, grid, block, 0, s, a.offset, a.top_k, a.scores, a.ld, a.idx);
}

}  // namespace dsa
