// sparse_mla.hip -- steps 3-7 of the DSA prefill path: attention of each query
// over only its selected latent rows (gather, QK^T, masked online softmax, PV,
// epilogue).
//
// For query i (absolute position p) and head h, over the slots t of idx[i]
// holding a key j with 0 <= j <= p:
//   l_t = sm_scale * <q[i][h], kv[j]>   (all d_latent + d_rope dims)
//   out[i][h] = sum_t softmax(l)_t * kv[j][0 : d_latent],  lse = log sum_t exp(l_t)
// (feedman.me page: the "DSA sparse-attention core" attends each query to its
// 2,048 gathered keys of the "512-wide latent KV"; the pages' own kernel runs
// one query per threadgroup with scalar dot products, and the same paragraph
// proposes using the matrix units -- which is what the fast kernel below does.)
//
// Fast kernel (bf16, 64 heads, 512 + 64 dims): one workgroup per query. The 64
// heads of one query share every gathered latent row, so they form the M = 64
// side of both products and no MFMA lane is wasted on masking. Per tile of 32
// selected slots:
//   gather  : each thread loads 16-byte pieces of the selected rows into
//             registers one tile ahead; the rows go to LDS twice -- key-major
//             for Q K^T and transposed (dim-major) for P V;
//   Q K^T   : wave w owns heads 16w..16w+15; S^T = K Q^T on 16x16x32 bf16
//             MFMAs with the query's Q fragments held in registers;
//   softmax : fp32, exp2 with log2(e) folded into the scale, running max and
//             sum per head; P goes to LDS as bf16 (split into hi + lo bf16
//             parts when the query has few valid keys, where single bf16
//             rounding of a large weight would show in the output);
//   P V     : wave w owns output dims 128w..128w+127 for all 64 heads.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

// ----------------------------------------------------------------- plain kernel

constexpr int kPlainThreads = 256;

__device__ __forceinline__ float act_load(const float* p, int64_t e) { return p[e]; }
__device__ __forceinline__ float act_load(const uint16_t* p, int64_t e) { return bf16_to_f32(p[e]); }

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += red[w];
  return r;
}

// grid = (n_q, n_heads). Any dims; fp32 arithmetic.
template <typename T>
__global__ __launch_bounds__(kPlainThreads) void mla_plain_kernel(int offset, int n_heads, int d_qk, int d_v,
                                                                  int top_k, float sm_scale,
                                                                  const T* __restrict__ q,
                                                                  const T* __restrict__ kv,
                                                                  const int32_t* __restrict__ idx,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse) {
  extern __shared__ float smem[];
  float* sq = smem;                                            // [d_qk]
  float* sw = sq + d_qk;                                       // [top_k] logits, then weights
  int32_t* sj = reinterpret_cast<int32_t*>(sw + top_k);        // [top_k] key or -1
  __shared__ float red[kPlainThreads / 64];
  const int i = blockIdx.x, h = blockIdx.y;
  const int64_t p = (int64_t)offset + i;
  const int64_t qbase = ((int64_t)i * n_heads + h) * d_qk;
  for (int d = threadIdx.x; d < d_qk; d += kPlainThreads) sq[d] = act_load(q, qbase + d);
  __syncthreads();
  float lmax = -INFINITY;
  for (int t = threadIdx.x; t < top_k; t += kPlainThreads) {
    const int32_t j = idx[(int64_t)i * top_k + t];
    const bool valid = j >= 0 && j <= p;
    float l = -INFINITY;
    if (valid) {
      float dot = 0.0f;
      for (int d = 0; d < d_qk; ++d) dot = fmaf(sq[d], act_load(kv, (int64_t)j * d_qk + d), dot);
      l = dot * sm_scale;
    }
    sw[t] = l;
    sj[t] = valid ? j : -1;
    lmax = fmaxf(lmax, l);
  }
  const float m = block_reduce_max(lmax, red);
  float* o = out + ((int64_t)i * n_heads + h) * d_v;
  if (m == -INFINITY) {
    for (int c = threadIdx.x; c < d_v; c += kPlainThreads) o[c] = 0.0f;
    if (lse && threadIdx.x == 0) lse[(int64_t)i * n_heads + h] = -INFINITY;
    return;
  }
  float lsum = 0.0f;
  for (int t = threadIdx.x; t < top_k; t += kPlainThreads) {
    const float e = sj[t] >= 0 ? expf(sw[t] - m) : 0.0f;
    sw[t] = e;
    lsum += e;
  }
  const float L = block_reduce_sum(lsum, red);  // its barriers also publish sw
  const float inv = 1.0f / L;
  for (int c = threadIdx.x; c < d_v; c += kPlainThreads) {
    float acc = 0.0f;
    for (int t = 0; t < top_k; ++t) {
      const int32_t j = sj[t];
      if (j >= 0) acc = fmaf(sw[t], act_load(kv, (int64_t)j * d_qk + c), acc);
    }
    o[c] = acc * inv;
  }
  if (lse && threadIdx.x == 0) lse[(int64_t)i * n_heads + h] = m + logf(L);
}

// ------------------------------------------------------------------ MFMA kernel

constexpr int kH = 64;              // heads
constexpr int kDL = 512;            // latent / value dims
constexpr int kDR = 64;             // rope dims
constexpr int kDQK = kDL + kDR;     // 576
constexpr int kTile = 32;           // selected slots per tile
constexpr int kThreads = 512;       // 8 waves (two per SIMD)
constexpr int kStages = 3;          // tiles resident in LDS (1 in use + 2 in flight)
constexpr int kRowBytes = kDQK * 2;              // 1152 = 72 pieces of 16 bytes
constexpr int kStageBytes = kTile * kRowBytes;   // 36 KB
constexpr int kMaxTopk = 4096;      // the whole index row lives in LDS
constexpr int kHiloMaxValid = 512;  // queries with at most this many valid keys use hi/lo P
constexpr float kRefLog2 = 64.0f;   // P = exp2(s - m_ref) < 2^64 before a restart is forced

// Max / sum over the four lanes l16 + 16*q (q = 0..3) that hold one head, with
// the gfx950 VALU lane swaps (xor-32, then xor-16 within each half).
__device__ __forceinline__ float max_over_q4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_q4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bool slot_valid(int32_t j, int64_t p) { return j >= 0 && (int64_t)j <= p; }

// Two fp32 -> packed bf16 pair (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

struct MlaSmem {
  uint8_t stage[kStages][kStageBytes];  // tiles: [32 rows][1 KB latent] then [32 rows][128 B rope]
  int32_t sidx[kMaxTopk];               // the query's slots: key, or -1 if not a valid key
  uint32_t tmask[kMaxTopk / kTile];     // validity bit per slot, one word per tile
  uint8_t pbuf[2][kH * kTile * 2];      // P (bf16, chunk-swizzled rows): hi part, lo part
  f32x4 sx[4][2][64];                   // Q K^T partial sums exchanged between the two k-halves
  float hmax[2][kH];                    // per key half: a head's max over the tile (reference exchange)
  float hsum[2][kH];                    // per key half: a head's row sum (epilogue)
  int32_t restart;                      // a head raised its reference: restart the query
  int last_slot;                        // one past the last valid slot
  int first_tile;                       // first tile holding a valid slot
  int n_valid;
};

// A stage holds the 32 rows of a tile as a 1 KB latent part per row (pieces
// 0..63, 8 dims each) followed by a 128-byte rope part per row (pieces
// 64..71). The LDS has 64 banks of 4 bytes, i.e. 16 positions of 16 bytes per
// bank cycle. Latent piece s of row r is stored at s ^ (r & 15) (the XOR stays
// within aligned groups of 16 pieces); rope piece s of row r at s ^ ((r >> 1) & 7).
// Both operand reads then spread over all banks: a Q K^T read (one piece of 16
// consecutive rows) and a transposed P V read (two pieces of 16 rows 8G + e).
constexpr int kLatBytes = 1024;
constexpr int kRopeOff = kTile * kLatBytes;  // 32 KB
__device__ __forceinline__ int swl(int r) { return r & 15; }
__device__ __forceinline__ int swr(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lat_off(int r, int s) { return r * kLatBytes + 16 * (s ^ swl(r)); }
__device__ __forceinline__ int rope_off(int r, int s) { return kRopeOff + r * 128 + 16 * (s ^ swr(r)); }
// P rows (one per head, 32 bf16 = 64 bytes = 4 chunks of 8 slots): chunk c of
// head h is stored at c ^ ((h >> 2) & 3), which keeps both the 8-byte softmax
// writes and the 16-byte operand reads free of bank conflicts.
__device__ __forceinline__ int p_off(int h, int c) { return h * 64 + 16 * (c ^ ((h >> 2) & 3)); }

// Waits until at most N vector-memory operations of this wave are in flight
// (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// then synchronises. Unlike __syncthreads() it does not drain the direct-to-LDS
// loads still in flight for later tiles; the tile about to be read is waited
// for explicitly with wait_vmcnt before this barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Eight transposed 64-bit LDS reads (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane j receives element j % 4 of the 4-element rows addressed by
// lanes 4e + j / 4 (e = 0..3). Written as one asm statement that also waits for
// the reads, so no read is in flight when the statement ends; the outputs are
// early-clobber so that no destination can overlap an address. (As a builtin,
// the compiler would drain the direct-to-LDS loads of later tiles before it.)
__device__ __forceinline__ void read_tr8(uint64_t (&d)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Direct-to-LDS loads of one tile: 36 blocks of 1 KB. Block m < 32 is the
// latent part of row m (lane L fills position L, i.e. loads piece L ^ (m & 15));
// block 32 + b holds the rope parts of rows 8b .. 8b+7 (lane L fills position
// L % 8 of row 8b + L/8, i.e. loads rope piece (L % 8) ^ swr(row)).
// Wave w issues the latent blocks 4w .. 4w+3, and waves 0-3 also rope block w.
// Slots whose key is not valid load the query's own row instead (always
// present, finite) and are masked in the softmax, so every tile costs a fixed
// number of loads per wave and the vmcnt bookkeeping stays exact. Addresses
// are 32-bit byte offsets from the cache base (the host checks that the cache
// is below 4 GiB). Each load is issued from asm: with the builtin, the compiler
// cannot tell which LDS reads alias the DMA and drains every load in flight
// before the next tile's operand reads. There is no register output to track;
// M0 is set here and used by nothing else in this kernel; completion is
// tracked with the explicit vmcnt waits of the tile loop.
__device__ __forceinline__ void dma16(const uint8_t* __restrict__ kv, uint32_t off, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(kv), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void issue_tile(MlaSmem& sm, const uint8_t* __restrict__ kv, int tile, int stage, int wave,
                                           int lane, uint32_t p) {
  const int32_t* sidx = sm.sidx + tile * kTile;
  const int32_t jl = sidx[lane & 31];                    // lane l: slot l % 32 (latent rows)
  const int rr = 8 * (wave & 3) + (lane >> 3);           // rope row of this lane
  const int32_t jr = sidx[rr];
  const uint32_t stage_lds = lds_addr(sm.stage[stage]);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = 4 * wave + u;
    const int32_t j = __builtin_amdgcn_readlane(jl, m);  // wave-uniform
    const uint32_t row = j >= 0 ? (uint32_t)j : p;
    dma16(kv, row * (uint32_t)kRowBytes + 16u * (uint32_t)(lane ^ swl(m)), stage_lds + kLatBytes * m);
  }
  if (wave < 4) {
    const uint32_t row = jr >= 0 ? (uint32_t)jr : p;
    dma16(kv, row * (uint32_t)kRowBytes + 2u * kDL + 16u * (uint32_t)((lane & 7) ^ swr(rr)),
          stage_lds + kRopeOff + 1024 * wave);
  }
}
// Waits until this wave's loads of the tile about to be read have landed,
// leaving the next tile's loads (if any) in flight.
__device__ __forceinline__ void wait_tile(int wave, bool next_in_flight) {
  if (!next_in_flight) wait_vmcnt<0>();
  else if (wave < 4) wait_vmcnt<5>();
  else wait_vmcnt<4>();
}

template <bool HILO>
__device__ __forceinline__ void pv_tile(f32x4 (&o)[4][4], const MlaSmem& sm, uint32_t tile_lds,
                                        const uint32_t (&tr_base)[8], int l16, int q4) {
  uint32_t a[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) a[x] = tile_lds + tr_base[x];  // x = 2 nb + h
  uint64_t d[8];
  read_tr8(d, a);
  bf16x8 vf[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    vf[nb] = __builtin_bit_cast(bf16x8, (u32x4{(uint32_t)d[2 * nb], (uint32_t)(d[2 * nb] >> 32), (uint32_t)d[2 * nb + 1],
                                               (uint32_t)(d[2 * nb + 1] >> 32)}));
#pragma unroll
  for (int part = 0; part < (HILO ? 2 : 1); ++part) {
    bf16x8 pa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      pa[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sm.pbuf[part] + p_off(16 * mb + l16, q4)));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mb], vf[nb], o[mb][nb], 0, 0, 0);
  }
}

// One workgroup (8 waves, two per SIMD) per query.
//   Q K^T : wave w = 4 kd + hg covers heads 16 hg .. +15, all 32 slots of the
//           tile, and the k-steps of parity kd (32 dims each); the two halves
//           are summed through LDS, after which wave w owns slots 16 kd .. +15;
//   P V   : wave w covers output dims 64 w .. +63 for all 64 heads.
__global__ __launch_bounds__(kThreads, 1) void mla_mfma_kernel(int n_q, int offset, int top_k, float scale_log2,
                                                               const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kv,
                                                               const int32_t* __restrict__ idx,
                                                               float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) MlaSmem sm;
  const int i = blockIdx.x;
  const int64_t p = (int64_t)offset + i;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3, kd = wave >> 2;  // head group; k-step parity, later key half
  const int l16 = lane & 15, q4 = lane >> 4;
  const int head = 16 * hg + l16;            // this lane's head in Q K^T / softmax
  const int32_t* __restrict__ idx_row = idx + (int64_t)i * top_k;
  const int n_slots = (top_k + kTile - 1) / kTile * kTile;
  const uint8_t* __restrict__ kvb = reinterpret_cast<const uint8_t*>(kv);

  // ---- stage the index row (invalid slots -> -1), per-tile validity masks.
  if (tid == 0) {
    sm.last_slot = 0;
    sm.n_valid = 0;
    sm.restart = 0;
    sm.first_tile = 0x7fffffff;
  }
  __syncthreads();
  {
    int last = 0, cnt = 0, first = 0x7fffffff;
    for (int t0 = 0; t0 < n_slots; t0 += kThreads) {
      const int t = t0 + tid;
      int32_t j = -1;
      if (t < top_k) j = idx_row[t];
      const bool ok = t < top_k && slot_valid(j, p);
      if (t < n_slots) sm.sidx[t] = ok ? j : -1;
      const uint64_t b = __ballot(ok);
      if (lane == 0 && t < n_slots) sm.tmask[t / kTile] = static_cast<uint32_t>(b);
      if (lane == 32 && t < n_slots) sm.tmask[t / kTile] = static_cast<uint32_t>(b >> 32);
      if (ok) {
        last = t + 1;
        first = min(first, t / kTile);
        ++cnt;
      }
    }
    last = (int)wave_max((float)last);  // exact: slots < 2^24
    cnt = wave_sum_int(cnt);
    first = -(int)wave_max(-(float)first);
    if (lane == 0) {
      atomicMax(&sm.last_slot, last);
      atomicAdd(&sm.n_valid, cnt);
      atomicMin(&sm.first_tile, first);
    }
  }

  // Q fragments (B operand of S^T = K Q^T): head 16 hg + l16, k-step 2u + kd,
  // dims 32 (2u + kd) + 8 q4 .. +7.
  bf16x8 qf[9];
  {
    const uint16_t* qsrc = q + ((int64_t)i * kH + head) * kDQK + 32 * kd + 8 * q4;
#pragma unroll
    for (int u = 0; u < 9; ++u) qf[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qsrc + 64 * u));
  }
  // Stage offsets of this lane's Q K^T operand pieces: piece 8u + 4kd + q4
  // (latent part for u < 8, rope part for u = 8) of row 16 kd + l16 (the slot
  // block this wave keeps, x = 0) and of row 16 (1 - kd) + l16 (the block it
  // hands over, x = 1). For u < 8 the swizzle depends on u only through u % 2,
  // so the address is qk_lat[x][u % 2] + 256 (u / 2).
  uint32_t qk_lat[2][2], qk_rope[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int row = 16 * (x == 0 ? kd : 1 - kd) + l16;
#pragma unroll
    for (int par = 0; par < 2; ++par) qk_lat[x][par] = lat_off(row, 8 * par + 4 * kd + q4);
    qk_rope[x] = rope_off(row, 4 * kd + q4);
  }
  // Transposed P V operand reads: lane 16G + s (s = 4e + c) addresses row
  // 8G + 4h + e, dims 64w + 16nb + 4c .. +3 (piece 8w + 2nb + c/2, byte
  // 8 (c % 2) inside it); entry x = 2 nb + h.
  uint32_t tr_base[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int nb = x >> 1, h = x & 1, e = l16 >> 2, c = l16 & 3;
    const int row = 8 * q4 + 4 * h + e;
    tr_base[x] = lat_off(row, 8 * wave + 2 * nb + (c >> 1)) + 8 * (c & 1);
  }
  __syncthreads();  // sidx, tmask, counts visible
  // Every load above (the Q fragments in particular) completes here, on every
  // path into the tile loop: inside the loop the only vector-memory operations
  // are the tile loads, whose count the explicit vmcnt waits rely on.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  const int n_tiles = (sm.last_slot + kTile - 1) / kTile;
  const int first_tile = sm.first_tile;
  const bool hilo = sm.n_valid <= kHiloMaxValid;
  const uint32_t p32 = (uint32_t)p;

  f32x4 o[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[mb][nb] = f32x4{0, 0, 0, 0};
  float m_ref = -INFINITY, l_part = 0.0f;  // this lane's head: reference (log2), partial sum

  if (n_tiles > 0) issue_tile(sm, kvb, 0, 0, wave, lane, p32);
  if (n_tiles > 1) issue_tile(sm, kvb, 1, 1, wave, lane, p32);
  // Each restart happens at a later tile than the previous one, so n_tiles
  // restarts always suffice; the cap only guarantees termination.
  int restarts_left = n_tiles;

  int st = 0;  // stage of tile t; tile t + 2 goes to stage (st + 2) % 3
  for (int t = 0; t < n_tiles; ++t, st = (st == kStages - 1) ? 0 : st + 1) {
    wait_tile(wave, t + 1 < n_tiles);
    lds_barrier();  // tile t resident for every wave; iteration t-1 finished everywhere
    if (t + 2 < n_tiles) issue_tile(sm, kvb, t + 2, st == 0 ? 2 : st - 1, wave, lane, p32);
    const uint8_t* __restrict__ tileb = sm.stage[st];

    // ---- partial S^T = K Q^T over this wave's k-steps, both 16-slot blocks.
    f32x4 sacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};  // [0] own block, [1] other block
#pragma unroll
    for (int u = 0; u < 9; ++u) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint8_t* src = (u < 8) ? tileb + qk_lat[x][u & 1] + 256 * (u >> 1) : tileb + qk_rope[x];
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src));
        sacc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[u], sacc[x], 0, 0, 0);
      }
      if (u == 4) __builtin_amdgcn_sched_barrier(0);  // bounds how far operand reads are hoisted
    }
    // Hand the other block's partial to the partner wave, add the partner's
    // partial of the own block.
    sm.sx[hg][1 - kd][lane] = sacc[1];
    lds_barrier();
    const f32x4 other = sm.sx[hg][kd][lane];
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = (sacc[0][r] + other[r]) * scale_log2;

    // ---- softmax for this lane's head over slots 16 kd + 4 q4 + r, in the
    // log2 domain, P = exp2(s - m_ref). m_ref is agreed by the two key-half
    // waves of the head at the first tile with a valid slot and may lag the
    // true maximum by up to kRefLog2, so P < 2^kRefLog2 (exact in relative
    // terms in bf16 and fp32) and the output accumulators are never rescaled
    // inside the loop. A logit beyond m_ref + kRefLog2 raises the reference and
    // restarts the query from its first tile with zeroed accumulators; each
    // restart happens at a later tile than the previous one.
    const uint32_t vb = sm.tmask[t];
    if (vb != 0xFFFFFFFFu) {  // partially valid tile (block-uniform)
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = ((vb >> (16 * kd + 4 * q4 + r)) & 1u) ? sv[r] : -INFINITY;
    }
    const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (t == first_tile) {  // block-uniform: agree on the references (one extra barrier per query)
      const float hm = max_over_q4(lmax);
      if (q4 == 0) sm.hmax[kd][head] = hm;
      lds_barrier();
      // Never lowers the reference: after a restart this tile is replayed and
      // the raised value must survive, or the restart would repeat.
      m_ref = fmaxf(m_ref, fmaxf(sm.hmax[0][head], sm.hmax[1][head]));
    } else if (__ballot(lmax > m_ref + kRefLog2) != 0) {
      if (max_over_q4(lmax) > m_ref + kRefLog2) sm.restart = 1;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;  // before the first valid tile: P = 0
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(sv[r] - m_use);
    l_part += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    {
      const uint32_t h0 = cvt_pk_bf16(pv[0], pv[1]);
      const uint32_t h1 = cvt_pk_bf16(pv[2], pv[3]);
      const int poff = p_off(head, 2 * kd + (q4 >> 1)) + 8 * (q4 & 1);  // slots 16 kd + 4 q4 .. +3
      *reinterpret_cast<u32x2*>(sm.pbuf[0] + poff) = u32x2{h0, h1};
      if (hilo) {
        const float r0 = pv[0] - __uint_as_float(h0 << 16), r1 = pv[1] - __uint_as_float(h0 & 0xFFFF0000u);
        const float r2 = pv[2] - __uint_as_float(h1 << 16), r3 = pv[3] - __uint_as_float(h1 & 0xFFFF0000u);
        *reinterpret_cast<u32x2*>(sm.pbuf[1] + poff) = u32x2{cvt_pk_bf16(r0, r1), cvt_pk_bf16(r2, r3)};
      }
    }
    lds_barrier();

    if (sm.restart && restarts_left > 0) {  // block-uniform (written before the barrier above); rare
      --restarts_left;
      const float hm = max_over_q4(lmax);
      if (q4 == 0) sm.hmax[kd][head] = hm;
      wait_vmcnt<0>();  // drain the loads of later tiles
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[mb][nb] = f32x4{0, 0, 0, 0};
      l_part = 0.0f;
      lds_barrier();  // flag read everywhere, maxima published; nobody reads a stage or P now
      m_ref = fmaxf(m_ref, fmaxf(sm.hmax[0][head], sm.hmax[1][head]));
      if (tid == 0) sm.restart = 0;
      issue_tile(sm, kvb, 0, 0, wave, lane, p32);
      if (n_tiles > 1) issue_tile(sm, kvb, 1, 1, wave, lane, p32);
      t = -1;
      st = kStages - 1;  // the loop increment brings it to stage 0 with t = 0
      continue;
    }
    // ---- O[64 heads][dims 64w..] += P V, V read straight from the tile's
    // latent part through transposed LDS reads.
    const uint32_t tile_lds = lds_addr(tileb);
    if (hilo) pv_tile<true>(o, sm, tile_lds, tr_base, l16, q4);
    else pv_tile<false>(o, sm, tile_lds, tr_base, l16, q4);
  }

  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2.
  const float lh = sum_over_q4(l_part);
  if (q4 == 0) sm.hsum[kd][head] = lh;
  __syncthreads();
  if (wave < 4 && q4 == 0) {
    const float l_run = sm.hsum[0][head] + sm.hsum[1][head];
    if (lse) lse[(int64_t)i * kH + head] = (l_run > 0.0f) ? (m_ref + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f : -INFINITY;
  }
  float* __restrict__ orow = out + (int64_t)i * kH * kDL;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 16 * mb + 4 * q4 + r;
      const float l_run = sm.hsum[0][hh] + sm.hsum[1][hh];
      f[r] = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        orow[(int64_t)(16 * mb + 4 * q4 + r) * kDL + 64 * wave + 16 * nb + l16] = o[mb][nb][r] * f[r];
  }
}

}  // namespace

bool mla_fast_path(const MlaArgs& a) {
  return a.bf16 && a.n_heads == kH && a.d_latent == kDL && a.d_rope == kDR && a.top_k <= kMaxTopk;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (mla_fast_path(a)) {
    const float scale_log2 = a.sm_scale * 1.44269504088896340736f;
    hipLaunchKernelGGL(mla_mfma_kernel, dim3(a.n_q), dim3(kThreads), 0, s, a.n_q, a.offset, a.top_k, scale_log2,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv), a.idx, a.out, a.lse);
    return hipGetLastError();
  }
  const int d_qk = a.d_latent + a.d_rope;
  const size_t lds = sizeof(float) * (size_t)d_qk + (sizeof(float) + sizeof(int32_t)) * (size_t)a.top_k;
  if (a.bf16)
    hipLaunchKernelGGL(mla_plain_kernel<uint16_t>, dim3(a.n_q, a.n_heads), dim3(kPlainThreads), lds, s, a.offset,
                       a.n_heads, d_qk, a.d_latent, a.top_k, a.sm_scale, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.kv), a.idx, a.out, a.lse);
  else
    hipLaunchKernelGGL(mla_plain_kernel<float>, dim3(a.n_q, a.n_heads), dim3(kPlainThreads), lds, s, a.offset,
                       a.n_heads, d_qk, a.d_latent, a.top_k, a.sm_scale, static_cast<const float*>(a.q),
                       static_cast<const float*>(a.kv), a.idx, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
