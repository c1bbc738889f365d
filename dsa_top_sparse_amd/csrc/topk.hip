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

// ---------------------------------------------------------------------------
// Filtered select for rows of at most 65,536 keys (16-bit candidate indices),
// several rows per CU. The row is never held whole: its first kFsSample keys
// give a threshold tau a margin below the k-th key's expected place, one
// streamed pass keeps the keys >= tau (in index order, in LDS; per key only a
// float compare and a count), and the exact select and the ordered emit then
// run over those candidates only. A workgroup needs about 29 KB of
// LDS and few registers, so five rows share a CU. If the sample misleads (fewer
// than k keys >= tau, or more than fit), the row is selected again without a
// threshold: a full histogram pass, then a compaction of the keys at or above
// the k-th key's top digit (or, if those do not fit either, every later step
// streamed from global memory). Same arithmetic and result on every path.
// Digits: bits 31..21 (11), 20..10 (11), 9..0 (10).
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

__global__ __launch_bounds__(kFsThreads) void topk_filter_kernel(int offset, int k, const float* __restrict__ scores,
                                                                 int64_t ld, int32_t* __restrict__ idx) {
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
    sm.low_or = 0u;  // OR / AND of the last 10 bits, gathered by the first refinement level
    sm.low_and = 0x3FFu;
  }
  lds_sync();

  // ---- threshold from the sample: its key of rank rs (a fifth above the
  // rank the k-th key is expected at, plus 16), to 22 bits.
  const int S = min(n, kFsSample);
  const uint32_t rs = static_cast<uint32_t>(
      min<int64_t>(S, (static_cast<int64_t>(k) * S * 6 + 5 * static_cast<int64_t>(n) - 1) / (5 * static_cast<int64_t>(n)) + 16));
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
  const uint32_t tau = (bs << 21) | (b2 << 10);

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

  uint32_t b1, above1, cnt1;
  if (cbase >= static_cast<uint32_t>(k) && cbase <= static_cast<uint32_t>(kFsCap)) {
    // Candidate scores to keys, the histogram of their top 22 bits relative
    // to tau's (the last bin collects everything 2,047 steps above), and the
    // OR / AND of the last 10 bits of the keys below that last bin.
    const int nc = static_cast<int>(cbase);
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
    return;
  }

  // ---- the sample misled: exact top digit from a full histogram pass (32-bit
  // counts, in the candidate area), then the candidates of that digit and
  // above (if they fit).
  fs_zero<false>(sm.ckey);
  __syncthreads();
  for (int base = 0; base < n; base += kFsSlice) {
    const f32x4 v = fs_load4(row, base, n);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (base + 4 * tid + e < n) fs_count<false>(sm.ckey, score_key(v[e]) >> 21);
  }
  __syncthreads();
  fs_bucket<false>(sm.ckey, sm, static_cast<uint32_t>(k), &b1, &above1, &cnt1, buf);
  const bool fits = above1 + cnt1 <= static_cast<uint32_t>(kFsCap);
  if (fits) {
    cbase = 0;
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
  if (tid == 0) {
    sm.low_or = 0u;
    sm.low_and = 0x3FFu;
  }
  __syncthreads();
  fs_tail(sm, buf, row, n, k, out, b1, 21, static_cast<uint32_t>(k) - above1, cnt1, false, fits,
          static_cast<int>(above1 + cnt1));
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
