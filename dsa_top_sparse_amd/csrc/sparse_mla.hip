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
constexpr int kThreads = 256;       // 4 waves
constexpr int kStages = 3;          // tiles resident in LDS (1 in use + 2 in flight)
constexpr int kRowBytes = kDQK * 2;              // 1152 = 72 pieces of 16 bytes
constexpr int kStageBytes = kTile * kRowBytes;   // 36 KB
constexpr int kDmaPerWave = kStageBytes / (1024 * (kThreads / 64));  // 9 x 1 KB per wave per tile
constexpr int kMaxTopk = 4096;      // the whole index row lives in LDS
constexpr int kHiloMaxValid = 512;  // queries with at most this many valid keys use hi/lo P
constexpr float kLazyLog2 = 8.0f;   // a head's reference max is raised only past +8 (log2)


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

struct MlaSmem {
  uint8_t stage[kStages][kStageBytes];  // key-major tiles, 16-byte pieces swizzled per row
  int32_t sidx[kMaxTopk];               // the query's slots: key, or -1 if not a valid key
  uint32_t tmask[kMaxTopk / kTile];     // validity bit per slot, one word per tile
  uint16_t pbuf[2][kH][kTile];          // P (bf16): hi part, lo part
  float alpha[kH];                      // per-head rescale of the running output
  int32_t rescale[4];                   // wave w raised a reference max of heads 16w.. this tile
  float fin[kH];                        // per-head 1 / l at the end
  int last_slot;                        // one past the last valid slot
  int n_valid;
};

// Piece s (0..71, 8 dims each) of tile row r is stored at piece s ^ swz(r).
// This swizzle spreads both operand reads evenly over the LDS banks: the Q K^T
// reads (one piece of 16 rows) and the transposed P V reads (two pieces of 16
// rows spaced 8G + e apart).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ (((r >> 3) & 3) << 1); }
__device__ __forceinline__ int piece_off(int r, int s) { return r * kRowBytes + 16 * (s ^ swz(r)); }

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

// Issues the direct-to-LDS loads of one tile: every wave writes 9 contiguous
// 1 KB blocks of the stage; lane L of block m fills 16-byte slot 64m + L, whose
// (row, piece) was precomputed in desc[]. Slots whose key is not valid load the
// query's own row instead (always present, finite) and are masked in the
// softmax, so every tile costs exactly kDmaPerWave loads per wave and the
// vmcnt bookkeeping stays exact.
__device__ __forceinline__ void issue_tile(MlaSmem& sm, const uint16_t* __restrict__ kv, int tile, int stage,
                                           const uint32_t* desc, int wave, int64_t p) {
  uint8_t* base = sm.stage[stage] + 1024 * (kDmaPerWave * wave);
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int r = desc[u] >> 8, piece = desc[u] & 0xFF;
    const int32_t j = sm.sidx[tile * kTile + r];
    const int64_t row = j >= 0 ? (int64_t)j : p;
    const uint16_t* src = kv + row * kDQK + 8 * piece;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + 1024 * u), 16, 0, 0);
  }
}

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
  const int l16 = lane & 15, q4 = lane >> 4;
  const int32_t* __restrict__ idx_row = idx + (int64_t)i * top_k;
  const int n_slots = (top_k + kTile - 1) / kTile * kTile;

  // ---- stage the index row (invalid slots -> -1), per-tile validity masks.
  if (tid == 0) {
    sm.last_slot = 0;
    sm.n_valid = 0;
  }
  __syncthreads();
  {
    int last = 0, cnt = 0;
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
        ++cnt;
      }
    }
    last = (int)wave_max((float)last);  // exact: slots < 2^24
    cnt = wave_sum_int(cnt);
    if (lane == 0) {
      atomicMax(&sm.last_slot, last);
      atomicAdd(&sm.n_valid, cnt);
    }
  }

  // Q fragments (B operand of S^T = K Q^T): head 16*wave + l16, dims 32ks + 8q4 .. +7.
  bf16x8 qf[kDQK / 32];
  {
    const uint16_t* qsrc = q + ((int64_t)i * kH + 16 * wave + l16) * kDQK + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < kDQK / 32; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qsrc + 32 * ks));
  }
  // This lane's DMA slots: slot P = 64 (9 wave + u) + lane -> (row, logical piece).
  uint32_t desc[kDmaPerWave];
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int P = 64 * (kDmaPerWave * wave + u) + lane;
    const int r = P / 72, pp = P - 72 * r;
    desc[u] = (uint32_t)(r << 8) | (uint32_t)(pp ^ swz(r));
  }
  __syncthreads();  // sidx, tmask, counts visible (also drains the loads above)
  const int n_tiles = (sm.last_slot + kTile - 1) / kTile;
  const bool hilo = sm.n_valid <= kHiloMaxValid;

  f32x4 o[4][8];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0, 0, 0, 0};
  float m_ref = -INFINITY, l_part = 0.0f;  // head 16*wave + l16: reference max, partial sum

  if (n_tiles > 0) issue_tile(sm, kv, 0, 0, desc, wave, p);
  if (n_tiles > 1) issue_tile(sm, kv, 1, 1, desc, wave, p);

  for (int t = 0; t < n_tiles; ++t) {
    const int st = t % kStages;
    if (t + 1 < n_tiles) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<0>();
    lds_barrier();  // tile t resident for every wave; iteration t-1 finished everywhere
    if (t + 2 < n_tiles) issue_tile(sm, kv, t + 2, (t + 2) % kStages, desc, wave, p);
    const uint8_t* __restrict__ tileb = sm.stage[st];

    // ---- S^T = K Q^T for this wave's 16 heads: two 16-slot blocks, each
    // accumulated in two independent chains (even / odd k-steps).
    f32x4 sacc[2][2] = {{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}, {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}};
#pragma unroll
    for (int ks = 0; ks < kDQK / 32; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tileb + piece_off(16 * mb + l16, 4 * ks + q4)));
        sacc[mb][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[mb][ks & 1], 0, 0, 0);
      }
    }
    f32x4 s[2] = {sacc[0][0] + sacc[0][1], sacc[1][0] + sacc[1][1]};
    // ---- softmax for head 16*wave + l16 over slots 16mb + 4q4 + r, in the
    // log2 domain. m_ref is the head's reference maximum: P = exp2(s - m_ref).
    // It is only raised when a logit exceeds it by more than kLazyLog2, so P
    // stays below 2^kLazyLog2 and the output rows need no rescaling on most
    // tiles (the rows of a head are rescaled only on the tiles that raise it).
    const uint32_t vb = sm.tmask[t];
    float lmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 16 * mb + 4 * q4 + r;
        const float v = ((vb >> slot) & 1u) ? s[mb][r] * scale_log2 : -INFINITY;
        s[mb][r] = v;
        lmax = fmaxf(lmax, v);
      }
    bool rescaled = false;
    float alpha = 1.0f;
    if (__ballot(lmax > m_ref + kLazyLog2) != 0) {  // wave-uniform: some head must raise its reference
      const float tmax = max_over_q4(lmax);
      if (tmax > m_ref + kLazyLog2) {
        alpha = (m_ref == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - tmax);  // O, l are 0 before the first key
        m_ref = tmax;
      }
      rescaled = __ballot(alpha != 1.0f) != 0;
      if (rescaled && q4 == 0) sm.alpha[16 * wave + l16] = alpha;
    }
    if (lane == 0) sm.rescale[wave] = rescaled ? 1 : 0;
    uint32_t phi[2][2], plo[2][2];
    float psum = 0.0f;
    const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;  // a tile with no valid slot yet: P = 0
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(s[mb][r] - m_use);
        psum += pv[r];
      }
      phi[mb][0] = pack_bf16x2(pv[0], pv[1]);
      phi[mb][1] = pack_bf16x2(pv[2], pv[3]);
      if (hilo) {
        float lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t hb = (r < 2 ? phi[mb][0] : phi[mb][1]) >> (16 * (r & 1));
          lo[r] = pv[r] - bf16_to_f32((uint16_t)(hb & 0xFFFFu));
        }
        plo[mb][0] = pack_bf16x2(lo[0], lo[1]);
        plo[mb][1] = pack_bf16x2(lo[2], lo[3]);
      }
    }
    l_part = l_part * alpha + psum;  // this lane's share of the head's sum
    {
      const int head = 16 * wave + l16;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int slot = 16 * mb + 4 * q4;
        *reinterpret_cast<u32x2*>(&sm.pbuf[0][head][slot]) = u32x2{phi[mb][0], phi[mb][1]};
        if (hilo) *reinterpret_cast<u32x2*>(&sm.pbuf[1][head][slot]) = u32x2{plo[mb][0], plo[mb][1]};
      }
    }
    lds_barrier();

    // ---- O[64 heads][dims 128w..] = alpha * O + P V. The V operand comes
    // straight from the key-major tile through transposed LDS reads: lane
    // 16G + s (s = 4e + c) points at row 8G + 4h + e, dims 4c..4c+3 of the
    // 16-dim block, and receives dims l16 of rows 8G + 4h + 0..3.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (sm.rescale[mb]) {  // heads 16mb.. belong to wave mb; rare after the first tile
        const f32x4 al = *reinterpret_cast<const f32x4*>(&sm.alpha[16 * mb + 4 * q4]);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[mb][nb] *= al;
      }
    }
    bf16x8 pa[4], pl[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      pa[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.pbuf[0][16 * mb + l16][8 * q4]));
      if (hilo) pl[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.pbuf[1][16 * mb + l16][8 * q4]));
    }
    const uint32_t tile_lds = lds_addr(tileb);
    const int s16 = lane & 15;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      uint32_t a[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int nb = 4 * blk + (x >> 1), h = x & 1;
        const int row = 8 * q4 + 4 * h + (s16 >> 2);
        const int col = 128 * wave + 16 * nb + 4 * (s16 & 3);  // first of 4 dims
        a[x] = tile_lds + row * kRowBytes + 16 * ((col >> 3) ^ swz(row)) + 2 * (col & 7);
      }
      uint64_t d[8];
      read_tr8(d, a);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int nb = 4 * blk + x;
        const u32x4 w = {(uint32_t)d[2 * x], (uint32_t)(d[2 * x] >> 32), (uint32_t)d[2 * x + 1],
                         (uint32_t)(d[2 * x + 1] >> 32)};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mb], vf, o[mb][nb], 0, 0, 0);
        if (hilo) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[mb], vf, o[mb][nb], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2.
  const float l_run = sum_over_q4(l_part);
  if (q4 == 0) {
    const int head = 16 * wave + l16;
    sm.fin[head] = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    if (lse) lse[(int64_t)i * kH + head] = (l_run > 0.0f) ? (m_ref + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f : -INFINITY;
  }
  __syncthreads();
  float* __restrict__ orow = out + (int64_t)i * kH * kDL;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const f32x4 f = *reinterpret_cast<const f32x4*>(&sm.fin[16 * mb + 4 * q4]);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        orow[(int64_t)(16 * mb + 4 * q4 + r) * kDL + 128 * wave + 16 * nb + l16] = o[mb][nb][r] * f[r];
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
