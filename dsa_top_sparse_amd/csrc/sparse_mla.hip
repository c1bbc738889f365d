// sparse_mla.hip -- steps 3-7 of the DSA prefill path: attention of each query
// over only its selected latent rows (gather, QK^T, masked online softmax, PV,
// epilogue).
//
// For query i (absolute position p) and head h, over the slots t of idx[i]
// holding a key j with 0 <= j <= p:
//   l_t = sm_scale * <q[i][h], kv[j]>   (all d_latent + d_rope dims)
//   out[i][h] = sum_t softmax(l)_t * kv[j][0 : d_latent],  lse = log sum_t exp(l_t)
// (feedman.me page, profile table row DSA sparse-attention core: each query
// attends to the 2,048 keys it gathered from the per-token latent cache, whose
// rows are 512 values wide; the pages' own kernel runs
// one query per threadgroup with scalar dot products, and the same paragraph
// proposes using the matrix units -- which is what the fast kernel below does.)
//
// Fast kernel (bf16, 64 heads, 512 + 64 dims): one workgroup of 8 waves per
// query. The 64 heads of one query share every gathered latent row, so they
// form the M = 64 side of both products and no MFMA lane is wasted on
// masking. Per tile of 32 selected slots:
//   gather  : all waves issue direct-to-LDS 16-byte loads of the selected
//             rows, two tiles ahead, into one of 4 LDS stages (latent parts
//             in four 8 KB groups of 128 dims, then the rope parts);
//   Q K^T   : score waves 0-3 each own 32 heads x 16 slots; S^T = K Q^T on
//             16x16x32 bf16 MFMAs with the query's Q fragments in registers;
//   softmax : fp32, exp2 with log2(e) folded into the scale, against a fixed
//             per-head reference (no running rescale); P goes to LDS as bf16
//             (split into hi + lo bf16 parts when the query has few valid
//             keys, where single bf16 rounding of a large weight would show);
//   P V     : P V waves 4-7 each own output dims 128v..128v+127 of all 64
//             heads, reading V transposed out of the stage.
// The two roles run side by side on every SIMD, one tile apart, and meet at
// one barrier per tile (details at the kernel).
#include <mutex>
#include <unordered_map>

#include "common.h"
#include "device_checks.h"
#include "kernels.h"

#include <type_traits>

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
  lds_poison(4u * (uint32_t)(d_qk + 2 * top_k));  // smem[]
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
static_assert(kTile == kDecodeTile, "decode splits are whole tiles");
constexpr int kThreads = 512;       // 8 waves: 4 score waves + 4 P V waves
constexpr int kStages = 4;          // LDS tile stages (hi/lo queries use 3; P's lo part takes the 4th)
constexpr int kRowBytes = kDQK * 2;              // 1152 = 72 pieces of 16 bytes
constexpr int kStageBytes = kTile * kRowBytes;   // 36 KB
constexpr int kOPad = 132;  // floats per head row of a P V wave's staged O (128 dims + 4: conflict-free writes)
static_assert(4 * kH * kOPad * 4 <= kStages * kStageBytes, "staged O of the 4 P V waves fits in the stages");
static_assert(kStageBytes % 256 == 0, "stage bases leave the low 8 address bits alone");
constexpr int kRingTiles = 32;      // index ring: 4 parts of 8 tiles (1 KB each)
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

// Two fp32 -> packed bf16 pair (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

struct MlaSmem {
  uint8_t stage[kStages][kStageBytes];  // tiles: [32 rows][1 KB latent] then [32 rows][128 B rope]
  uint8_t pbuf[2][kH * kTile * 2];      // P hi part (bf16, chunk-swizzled rows) by tile parity
  int32_t ring[kRingTiles][kTile];      // the query's index row, tile t at t % 32
  float hmax[2][kH];                    // [slot half][head]: maxima exchanged between the slot halves
  float lsum[2][kH];                    // [slot half][head]: softmax denominators at the end
  int32_t restart;                      // a head passed its reference by more than kRefLog2
  int32_t c_last, c_valid, c_first;     // index row census
  int32_t c_firstbad;                   // first tile with a slot that is not a causal key
};

// A stage holds the latent parts of the tile's 32 rows as 4 groups of 8 KB
// (group g: pieces 16g .. 16g+15, i.e. dims 128g .. 128g+127, of every row, as
// [32 rows][256 bytes]) followed by the rope parts as [32 rows][128 bytes]
// (rope pieces 64..71). The LDS has 64 banks of 4 bytes, i.e. 16 positions of
// 16 bytes per bank cycle, and every row of a group starts a bank cycle.
// Latent piece 16g + s of row r is stored at position s ^ swl(r) of its row
// in group g; rope piece s of row r at s ^ ((r >> 1) & 7).
// swl is the linear map of the row's low four bits b0..b3 that sends b0 to 4,
// b1 to 8, b2 to 2 and b3 to 3 (XOR-combined). Both operand reads are then
// free of bank conflicts, as the LDS bank-conflict counter shows for their
// exact address patterns:
//  - a Q K^T read (16-byte reads, one piece of 16 consecutive rows per
//    quarter wave); the plain map swl(r) = r & 15 is conflict-free here too,
//    but other one-to-one maps, e.g. the bit permutation 2, 4, 1, 8, are not:
//    the hardware does not serve a 16-byte read as four quarter waves;
//  - a transposed P V read (8 bytes per lane; pieces 2n, 2n + 1 of rows
//    8G + 4h + e): swl(r) >> 1 differs for the eight rows (G, e) that one
//    half wave reads, so the second piece cannot collide. With r & 15, rows
//    e and e ^ 1 took the same two positions (two-way conflicts).
// The group-major order lets one 1 KB direct-to-LDS load fill a group of four
// consecutive rows (64 lanes x 16 bytes land contiguously), so a wave fills
// its four rows with four loads that differ only in immediate offsets.
constexpr int kGroupBytes = kTile * 256;      // 8 KB
constexpr int kRopeOff = 4 * kGroupBytes;     // 32 KB
__device__ __forceinline__ int swl(int r) { return (((r & 3) << 2) | ((r >> 1) & 2)) ^ (((r >> 3) & 1) * 3); }
__device__ __forceinline__ int swr(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lat_off(int r, int s) { return (s >> 4) * kGroupBytes + r * 256 + 16 * ((s & 15) ^ swl(r)); }
__device__ __forceinline__ int rope_off(int r, int s) { return kRopeOff + r * 128 + 16 * (s ^ swr(r)); }
// P rows (one per head, 32 bf16 = 64 bytes = 4 chunks of 8 slots): chunk c of
// head h is stored at c ^ ((h >> 2) & 3), which keeps the 16-byte operand
// reads free of bank conflicts (the two 8-byte softmax writes per tile and
// score wave still take two-way conflicts, a few cycles per tile).
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
// loads still in flight for later tiles; a tile about to be read is waited for
// explicitly with wait_vmcnt before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
__device__ __forceinline__ u32x4 lds_read16(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((lds_u8*)(uintptr_t)a);
}
__device__ __forceinline__ void lds_write8(uint32_t a, u32x2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((__attribute__((address_space(3))) uint8_t*)(uintptr_t)a) = v;
}
__device__ __forceinline__ s16x4 lds_read_tr(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_u8*)(uintptr_t)a));
}

// One direct-to-LDS load: 16 bytes per lane from base + off + IMM to LDS
// address lds + 16 * lane. The instruction's immediate offset applies to both
// the global and the LDS address, so M0 is set to lds - IMM. Issued from asm: with the builtin, the compiler cannot tell
// which LDS reads alias the load and drains every load in flight before the
// next tile's operand reads. There is no register output to track; M0 is set
// here and used by nothing else in this kernel; completion is tracked with the
// explicit vmcnt waits of the tile loop.
template <int IMM = 0>
__device__ __forceinline__ void dma16(const void* __restrict__ base, uint32_t off, uint32_t lds) {
  static_assert(IMM >= 0 && IMM < 4096, "immediate offset range");
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(off), "s"(base), "i"(IMM), "{m0}"(lds - IMM));
#pragma clang diagnostic pop
}

// Byte offset of a selected row in the cache. A slot holding no causal key
// (j < 0 or j > p, both above p as unsigned) loads the query's own row
// instead (always present, finite); so does, possibly, a slot past top_k,
// whose ring entry is some entry of the row. Such slots are masked in the
// softmax, so that every tile costs a fixed number of loads. The offsets are
// 32-bit (the host checks that the cache is below 4 GiB).
__device__ __forceinline__ uint32_t row_off(int32_t j, uint32_t p) {
  return min((uint32_t)j, p) * (uint32_t)kRowBytes;
}

// Tile loads, spread over all 8 waves: wave w loads the latent parts of the
// rows of slots 4w .. 4w+3, one load per group g (lane L fills position L % 16
// of row 4w + L / 16 in group g, i.e. loads latent piece 16g + (L % 16) ^
// swl(row)), and waves 0-3 also the rope parts of rows 8w .. 8w+7 (one load;
// lane L fills position L % 8 of row 8w + L / 8, i.e. loads rope piece
// (L % 8) ^ swr(row)). Per tile: 5 loads for waves 0-3, 4 for waves 4-7.
struct GatherRows {
  uint32_t lat;   // cache offset of this lane's latent bytes, group 0
  uint32_t rope;  // cache offset of this lane's rope bytes (waves 0-3)
};
// Lane constants of the gather: the slot whose row a lane loads and its
// byte position inside that row's group (latent) or rope part.
struct GatherLane {
  int sl, sr;            // latent slot 4w + L / 16, rope slot 8 (w % 4) + L / 8
  uint32_t lat, rope;    // byte offsets inside the cache row
};
__device__ __forceinline__ GatherLane gather_lane(int wave, int lane) {
  GatherLane gl;
  gl.sl = 4 * wave + (lane >> 4);
  gl.sr = 8 * (wave & 3) + (lane >> 3);
  gl.lat = 16u * (uint32_t)((lane & 15) ^ swl(gl.sl));
  gl.rope = 2u * kDL + 16u * (uint32_t)((lane & 7) ^ swr(gl.sr));
  return gl;
}
__device__ __forceinline__ GatherRows gather_rows(const int32_t* ring_tile, const GatherLane& gl, uint32_t p) {
  GatherRows g;
  g.lat = row_off(ring_tile[gl.sl], p) + gl.lat;
  g.rope = row_off(ring_tile[gl.sr], p) + gl.rope;
  return g;
}
// Load u of a tile for wave w: u < 4 latent group u; u = 4 the rope block
// (waves 0-3 only: the caller knows its role). u is a constant wherever this
// is called (unrolled loops), so the switch folds away.
__device__ __forceinline__ void gather_load(const uint8_t* __restrict__ kv, const GatherRows& g, uint32_t stage_lds,
                                            int u, int wave) {
  const uint32_t lds = stage_lds + (uint32_t)(1024 * wave);
  switch (u) {
    case 0: dma16<0>(kv, g.lat, lds); break;
    case 1: dma16<256>(kv, g.lat, lds + kGroupBytes); break;
    case 2: dma16<512>(kv, g.lat, lds + 2 * kGroupBytes); break;
    case 3: dma16<768>(kv, g.lat, lds + 3 * kGroupBytes); break;
    default: dma16(kv, g.rope, lds + kRopeOff); break;
  }
}

// Index ring refill: tiles 8c .. 8c+7 of the index row (1 KB) into ring part
// c % 4. Lanes whose 16 bytes would pass the end of the row read the row's
// last 16 bytes instead; their slots lie past top_k and are never used.
__device__ __forceinline__ void issue_ring(MlaSmem& sm, const int32_t* __restrict__ idx_row, int c, int top_k,
                                           int lane) {
  int s0 = 256 * c + 4 * lane;
  if (s0 + 4 > top_k) s0 = top_k - 4;
  dma16(idx_row, 4u * (uint32_t)s0, lds_addr(sm.ring[8 * (c & 3)]));
}

// One workgroup (8 waves, two per SIMD) per query, in two roles that run side
// by side on every SIMD and meet at one barrier per tile:
//   score waves (w = 0..3; g = w & 1, s = w >> 1): S^T = K Q^T for heads
//     32 g .. +31 and slots 16 s .. +15 of a tile over all 576 dims (the
//     query's Q fragments for those heads stay in registers), then the
//     softmax of those scores; P goes to LDS as bf16;
//   P V waves (w = 4..7; v = w - 4): O += P V for output dims 128 v .. +127
//     of all 64 heads.
// All waves share the direct-to-LDS tile loads, which each wave issues right
// after the barrier, before its products: the earlier they leave, the more of
// the gather latency the tile in between covers (issuing them between the
// products instead left the score waves waiting about 500 cycles per tile for
// their last rows).
// In iteration t the score waves work on tile t and the P V waves on tile
// t - 1, while tiles t + 1 and t + 2 are loading (4 stages).
//
// The softmax needs no running rescale: every head gets a fixed reference
// m_ref (log2 domain), its maximum over the first tile with a valid slot
// (the two slot halves agree on it through LDS in that iteration), and
// P = exp2(s - m_ref). The score waves track the largest s - m_ref; if a
// head's passed kRefLog2 (P could leave the range in which the fp32 sums
// stay accurate), the query is computed once more with each head's
// reference raised to its maximum.
//
// Split launch (gridDim.y > 1): workgroup (x, y) handles slots
// [y * split_slots, +split_slots) of the query's index row as if they were
// the whole row, and writes its normalised output and lse to slot y of the
// partial arrays (out / lse of shape [splits][n_q][...]); a combine kernel
// merges the splits.
__global__ __launch_bounds__(kThreads, 1) void mla_mfma_kernel(int n_q, int offset, int row_slots, int split_slots,
                                                               float scale_log2, const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kv,
                                                               const int32_t* __restrict__ idx,
                                                               float* __restrict__ out, float* __restrict__ lse) {
  lds_poison();
  __shared__ __attribute__((aligned(1024))) MlaSmem sm;
  const int i = n_q - 1 - (int)blockIdx.x;  // latest queries (most keys) first
  const int split = blockIdx.y;
  const int top_k = min(split_slots, row_slots - split * split_slots);  // slots of this workgroup
  const int64_t out_row = (int64_t)split * n_q + i;
  const uint32_t p32 = (uint32_t)(offset + i);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int32_t* __restrict__ idx_row = idx + (int64_t)i * row_slots + (int64_t)split * split_slots;
  const uint8_t* __restrict__ kvb = reinterpret_cast<const uint8_t*>(kv);
  uint32_t stage0_lds = lds_addr(sm.stage[0]);
  uint32_t pbuf_lds = lds_addr(sm.pbuf[0]);
  uint32_t plo_lds = lds_addr(sm.stage[kStages - 1]);  // P lo parts (hi/lo queries)
  // Held in scalar registers from here on (otherwise the compiler recomputes
  // the address-space conversions inside the tile loops).
  asm volatile("" : "+s"(stage0_lds), "+s"(pbuf_lds), "+s"(plo_lds));
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const GatherLane gl = gather_lane(wave, lane);

  if (tid == 0) {
    sm.c_last = 0;
    sm.c_valid = 0;
    sm.c_first = 0x7fffffff;
    sm.c_firstbad = (top_k % kTile) ? top_k / kTile : 0x7fffffff;  // a partial last tile is masked
    sm.restart = 0;
  }
  __syncthreads();

  // Census of the index row (valid slots, last valid slot, first tile with a
  // valid slot), then the tile range. Called by both roles after they have
  // issued their own first loads, so that the latencies overlap.
  int n_tiles = 0, first_tile = 0, t0 = 0, first_bad = 0;
  bool hilo = false;
  auto census = [&]() {
    int last = 0, cnt = 0, first = 0x7fffffff, bad = 0x7fffffff;
    for (int b = 4 * tid; b < top_k; b += 4 * kThreads) {  // top_k % 4 == 0: 16-byte reads
      const u32x4 j4 = *reinterpret_cast<const u32x4*>(idx_row + b);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (j4[r] <= p32) {  // 0 <= j <= p (negative j compare as large)
          last = b + r + 1;
          first = min(first, (b + r) / kTile);
          ++cnt;
        } else {
          bad = min(bad, (b + r) / kTile);
        }
      }
    }
    last = wave_max_int(last);
    cnt = wave_sum_int(cnt);
    first = wave_min_int(first);
    bad = wave_min_int(bad);
    if (lane == 0) {
      atomicMax(&sm.c_last, last);
      atomicAdd(&sm.c_valid, cnt);
      atomicMin(&sm.c_first, first);
      atomicMin(&sm.c_firstbad, bad);
    }
    if (wave == 7) {  // index ring, tiles 0..15 (reloaded below if the first valid tile lies further)
      issue_ring(sm, idx_row, 0, top_k, lane);
      issue_ring(sm, idx_row, 1, top_k, lane);
    }
    // Every load so far completes here: inside the tile loop the only
    // vector-memory operations are the tile and ring loads, whose counts the
    // explicit vmcnt waits rely on.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    n_tiles = (sm.c_last + kTile - 1) / kTile;
    first_tile = n_tiles > 0 ? sm.c_first : 0;
    first_bad = sm.c_firstbad;
    t0 = first_tile & ~7;  // the loop starts at a ring chunk boundary
    hilo = sm.c_valid <= kHiloMaxValid;
    if (t0 != 0) {  // rare: no valid slot in tiles 0..7
      if (wave == 7) {
        issue_ring(sm, idx_row, t0 / 8, top_k, lane);
        issue_ring(sm, idx_row, t0 / 8 + 1, top_k, lane);
        wait_vmcnt<0>();
      }
      __syncthreads();
    }
  };

  // Waits, before the barrier of iteration t, for this wave's loads of tile
  // t: only the loads of tile t + 1, the last ones this wave issued, may stay
  // in flight (a ring refill, issued before them, completes here too).
  // STEADY: t + 1 < n_tiles is known.
  auto wait_tile = [&](int t, auto hilo_c, auto steady_c) {
    constexpr bool HILO = decltype(hilo_c)::value;
    constexpr bool STEADY = decltype(steady_c)::value;
    if (!STEADY && t >= n_tiles) return;
    if (HILO || (!STEADY && t + 1 >= n_tiles)) {  // HILO: tile t + 1 is issued after this barrier
      wait_vmcnt<0>();
    } else if (wave < 4) {
      wait_vmcnt<5>();
    } else {
      wait_vmcnt<4>();
    }
  };
  auto issue_all = [&](const GatherRows& g, uint32_t stage_lds) {
#pragma unroll
    for (int u = 0; u < 4; ++u) gather_load(kvb, g, stage_lds, u, wave);
    if (wave < 4) gather_load(kvb, g, stage_lds, 4, wave);
  };
  auto start_pipeline = [&](int ahead) {
    for (int a = 0; a < ahead; ++a)
      if (t0 + a < n_tiles)
        issue_all(gather_rows(sm.ring[(t0 + a) & (kRingTiles - 1)], gl, p32),
                  stage0_lds + kStageBytes * a);
  };

  // ================================================================ score waves
  auto score_role = [&](auto hilo_c, const bf16x8 (&qf)[2][18]) {
    constexpr bool HILO = decltype(hilo_c)::value;
    constexpr int S = HILO ? kStages - 1 : kStages;
    constexpr int kAhead = S - 2;
    const int g = wave & 1, s = wave >> 1;
    int head[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) head[hb] = 32 * g + 16 * hb + l16;
    // K operand (A): row 16 s + l16 of the tile, piece 4u + q4. For u < 16 the
    // piece lies in group u / 4, so the offset is qk_lat[u % 4] + 8 KB (u / 4);
    // the rope k-steps u = 16, 17 have their own.
    const int krow = 16 * s + l16;
    uint32_t qk_lat[4], qk_rope[2];
#pragma unroll
    for (int x = 0; x < 4; ++x) qk_lat[x] = lat_off(krow, 4 * x + q4);
#pragma unroll
    for (int x = 0; x < 2; ++x) qk_rope[x] = rope_off(krow, 4 * x + q4);
    // A logit in log2 units. The product is rounded on its own and never
    // fused into a following subtraction, so that the maximal logit of the
    // reference tile gives exactly 0 - and P = 1 - wherever it is computed.
    auto scaled = [&](float acc) {
#pragma clang fp contract(off)
      return acc * scale_log2;
    };
    // P write position of this lane's 4 slots 16 s + 4 q4 .. +3 in each head row.
    uint32_t poff[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) poff[hb] = p_off(head[hb], 2 * s + (q4 >> 1)) + 8 * (q4 & 1);

    float m_ref[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.0f, 0.0f}, runmax[2] = {-INFINITY, -INFINITY};

    // Ring entries used in iteration t (the rows of tile t + kAhead, the slot
    // indices of tile t) are read in iteration t - 1, so that no LDS read
    // latency sits between the barrier and the first operand reads.
    auto ring_rows = [&](int t) {
      const int tn = t + kAhead;
      return gather_rows(sm.ring[(tn < n_tiles ? tn : t0) & (kRingTiles - 1)], gl, p32);
    };
    auto ring_slots = [&](int t) {
      return *reinterpret_cast<const u32x4*>(&sm.ring[t & (kRingTiles - 1)][16 * s + 4 * q4]);
    };
    auto pass = [&](const bf16x8 (&qf)[2][18], bool first_pass) {
      start_pipeline(kAhead);
      int st = 0;  // stage of tile t
      GatherRows rows = ring_rows(t0);
      u32x4 jv = ring_slots(t0);
      // One iteration; STEADY: first_tile < t and t + kAhead < n_tiles.
      auto body = [&](int t, auto steady_c) {
        constexpr bool STEADY = decltype(steady_c)::value;
        wait_tile(t, hilo_c, steady_c);
        lds_barrier();  // B(t): tile t resident; P(t - 1) complete
        const bool more = STEADY || t + kAhead < n_tiles;
        int sn = st + kAhead;
        if (sn >= S) sn -= S;
        const uint32_t next_lds = stage0_lds + kStageBytes * sn;
        GatherRows rows_n;
        u32x4 jv_n;
        if (STEADY || (t < n_tiles && t >= first_tile)) {
          // ---- tile t + kAhead's loads, then S^T = K Q^T
          if (more) issue_all(rows, next_lds);
          const uint32_t tile_lds = stage0_lds + kStageBytes * st;
          uint32_t kb[6];
#pragma unroll
          for (int x = 0; x < 4; ++x) kb[x] = tile_lds + qk_lat[x];
#pragma unroll
          for (int x = 0; x < 2; ++x) kb[4 + x] = tile_lds + qk_rope[x];
          // The operand reads run six k-steps ahead.
          auto kread = [&](int u) {
            return __builtin_bit_cast(bf16x8,
                                      lds_read16((u < 16) ? kb[u & 3] + kGroupBytes * (u >> 2) : kb[4 + (u - 16)]));
          };
          f32x4 sacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
          constexpr int kLead = 6;
          bf16x8 kf[kLead];
#pragma unroll
          for (int x = 0; x < kLead; ++x) kf[x] = kread(x);
#pragma unroll
          for (int u = 0; u < 18; ++u) {
            const bf16x8 cur = kf[u % kLead];
            if (u + kLead < 18) kf[u % kLead] = kread(u + kLead);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
              sacc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qf[hb][u], sacc[hb], 0, 0, 0);
          }
          rows_n = ring_rows(t + 1);
          jv_n = jv;
          if (t + 1 >= first_bad) jv_n = ring_slots(t + 1);
          // ---- slot validity and softmax numerators. Tiles before the first
          // one holding a non-causal slot (every tile, for an index row that
          // lists causal keys and then pads) need no masks.
          auto softmax = [&](auto masked_c) {
            constexpr bool MASKED = decltype(masked_c)::value;
            bool vm[4] = {true, true, true, true};
            if (MASKED) {
              const int gs0 = t * kTile + 16 * s + 4 * q4;
#pragma unroll
              for (int r = 0; r < 4; ++r) vm[r] = gs0 + r < top_k && jv[r] <= p32;
            }
            if (!STEADY && first_pass && t == first_tile) {  // reference: the head's max over this tile
#pragma unroll
              for (int hb = 0; hb < 2; ++hb) {
                float lm = -INFINITY;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (vm[r]) lm = fmaxf(lm, scaled(sacc[hb][r]));
                const float hm = max_over_q4(lm);
                if (q4 == 0) sm.hmax[s][head[hb]] = hm;
              }
              lds_barrier();  // X: both slot halves' maxima published
#pragma unroll
              for (int hb = 0; hb < 2; ++hb) m_ref[hb] = fmaxf(sm.hmax[0][head[hb]], sm.hmax[1][head[hb]]);
            }
            // P = exp2(s * scale - m_ref), bf16 to LDS (the product is rounded
            // as in the reference, so its maximum gets P = 1 exactly)
            const uint32_t par = (uint32_t)(t & 1) * (kH * kTile * 2);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              float x[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) x[r] = (!MASKED || vm[r]) ? scaled(sacc[hb][r]) - m_ref[hb] : -INFINITY;
              runmax[hb] = fmaxf(runmax[hb], fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
              float pv[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(x[r]);
              l_part[hb] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
              const uint32_t h0 = cvt_pk_bf16(pv[0], pv[1]);
              const uint32_t h1 = cvt_pk_bf16(pv[2], pv[3]);
              lds_write8(pbuf_lds + par + poff[hb], u32x2{h0, h1});
              if (HILO) {
                const float r0 = pv[0] - __uint_as_float(h0 << 16), r1 = pv[1] - __uint_as_float(h0 & 0xFFFF0000u);
                const float r2 = pv[2] - __uint_as_float(h1 << 16), r3 = pv[3] - __uint_as_float(h1 & 0xFFFF0000u);
                lds_write8(plo_lds + par + poff[hb], u32x2{cvt_pk_bf16(r0, r1), cvt_pk_bf16(r2, r3)});
              }
            }
          };
          if (t >= first_bad) softmax(std::true_type{});
          else softmax(std::false_type{});
        } else {
          if (more) issue_all(rows, next_lds);
          rows_n = ring_rows(t + 1);
          jv_n = ring_slots(t + 1);
        }
        rows = rows_n;
        jv = jv_n;
        st = (st + 1 == S) ? 0 : st + 1;
      };
      for (int t = t0; t <= n_tiles; ++t) {
        if (t > first_tile && t + kAhead < n_tiles) body(t, std::true_type{});
        else body(t, std::false_type{});
      }
    };

    pass(qf, true);
    // ---- did a head's scores pass its reference by more than kRefLog2?
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float hm = max_over_q4(runmax[hb]);
      if (q4 == 0) sm.hmax[s][head[hb]] = hm;
    }
    if (__ballot(runmax[0] > kRefLog2 || runmax[1] > kRefLog2) != 0) sm.restart = 1;
    lds_barrier();  // Z
    if (sm.restart) {  // block-uniform; rare
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        m_ref[hb] += fmaxf(sm.hmax[0][head[hb]], sm.hmax[1][head[hb]]);
        l_part[hb] = 0.0f;
      }
      lds_barrier();  // Z2: ring reloaded
      pass(qf, false);
    }
    // ---- epilogue: denominators to the P V waves; lse = (m + log2 l) * ln 2.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float lh = sum_over_q4(l_part[hb]);
      if (q4 == 0) sm.lsum[s][head[hb]] = lh;
    }
    wait_vmcnt<0>();  // no tile load in flight: the P V waves reuse the stages for O
    __syncthreads();  // E1
    if (lse && s == 0 && q4 == 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float l_run = sm.lsum[0][head[hb]] + sm.lsum[1][head[hb]];
        lse[out_row * kH + head[hb]] =
            (l_run > 0.0f) ? (m_ref[hb] + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f : -INFINITY;
      }
    }
  };

  // ================================================================= P V waves
  auto pv_role = [&](auto hilo_c) {
    constexpr bool HILO = decltype(hilo_c)::value;
    constexpr int S = HILO ? kStages - 1 : kStages;
    constexpr int kAhead = S - 2;
    const int v = wave - 4;
    // Transposed V reads (B operand): lane 16G + 4e + c addresses row
    // 8G + 4h + e, dims 128v + 16nb + 4c .. +3 (piece 16v + 2nb + c/2, byte
    // 8 (c % 2) inside it). The piece's position is 2nb ^ ((c / 2) ^ swl(row)),
    // so the address for dim block nb is tr_base[h] ^ 32 nb (the stage base,
    // a multiple of 256, does not touch those bits).
    uint32_t tr_base[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = l16 >> 2, c = l16 & 3;
      tr_base[h] = lat_off(8 * q4 + 4 * h + e, 16 * v + (c >> 1)) + 8 * (c & 1);
    }
    // P operand (A): head 16 mb + l16, slots 8 q4 .. +7; the head block adds 1 KB.
    const uint32_t pr = (uint32_t)p_off(l16, q4);
    f32x4 o[4][8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0, 0, 0, 0};

    auto ring_rows = [&](int t) {  // read one iteration ahead, as in the score waves
      const int tn = t + kAhead;
      return gather_rows(sm.ring[(tn < n_tiles ? tn : t0) & (kRingTiles - 1)], gl, p32);
    };
    auto pass = [&](bool first_pass) {
      start_pipeline(kAhead);
      int st = 0;  // stage of tile t
      GatherRows rows = ring_rows(t0);
      // (One loop body: two specialised copies, as in the score waves, would
      // each need their own registers for the 128 accumulators.)
      for (int t = t0; t <= n_tiles; ++t) {
        wait_tile(t, hilo_c, std::false_type{});
        lds_barrier();  // B(t)
        if (wave == 7 && (t & 7) == 0 && t >= t0 + 8 && 8 * (t / 8 + 1) < n_tiles)
          issue_ring(sm, idx_row, t / 8 + 1, top_k, lane);
        const bool more = t + kAhead < n_tiles;
        int sn = st + kAhead;
        if (sn >= S) sn -= S;
        const uint32_t next_lds = stage0_lds + kStageBytes * sn;
        GatherRows rows_n;
        if (t - 1 >= first_tile) {
          // ---- tile t + kAhead's loads, then O += P V for tile t - 1
          if (more) issue_all(rows, next_lds);
          const uint32_t tile_lds = stage0_lds + kStageBytes * (st == 0 ? S - 1 : st - 1);
          const uint32_t par = (uint32_t)((t - 1) & 1) * (kH * kTile * 2);
          // V operand reads run two dim blocks ahead.
          auto vread = [&](int nb) {
            const s16x4 d0 = lds_read_tr((tile_lds + tr_base[0]) ^ (uint32_t)(32 * nb));
            const s16x4 d1 = lds_read_tr((tile_lds + tr_base[1]) ^ (uint32_t)(32 * nb));
            return __builtin_bit_cast(bf16x8, (s16x8{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]}));
          };
#pragma unroll
          for (int part = 0; part < (HILO ? 2 : 1); ++part) {
            const uint32_t pb = (part ? plo_lds : pbuf_lds) + par + pr;
            bf16x8 pa[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) pa[mb] = __builtin_bit_cast(bf16x8, lds_read16(pb + 1024 * mb));
            bf16x8 vf[2] = {vread(0), vread(1)};
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
              const bf16x8 cur = vf[nb & 1];
              if (nb + 2 < 8) vf[nb & 1] = vread(nb + 2);
#pragma unroll
              for (int mb = 0; mb < 4; ++mb)
                o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mb], cur, o[mb][nb], 0, 0, 0);
              if (part == 0 && nb == 5) rows_n = ring_rows(t + 1);
              // keep the reads two dim blocks ahead, not all at the top (registers)
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else {
          if (more) issue_all(rows, next_lds);
          rows_n = ring_rows(t + 1);
        }
        rows = rows_n;
        // X: the score waves' reference exchange (same condition as theirs)
        if (first_pass && t == first_tile && t < n_tiles) lds_barrier();
        st = (st + 1 == S) ? 0 : st + 1;
      }
    };

    pass(true);
    lds_barrier();  // Z
    if (sm.restart) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0, 0, 0, 0};
      if (wave == 7) {
        issue_ring(sm, idx_row, t0 / 8, top_k, lane);
        issue_ring(sm, idx_row, t0 / 8 + 1, top_k, lane);
        wait_vmcnt<0>();
      }
      lds_barrier();  // Z2
      pass(false);
    }
    // ---- epilogue: O / l, staged through LDS so that every store writes
    // whole 128-byte lines. A lane holds one dim of four heads (16 lanes: 64
    // contiguous bytes of a head row); through the stages, which no wave reads
    // or loads after E1, each lane stores 4 consecutive dims of one head, and
    // one store instruction two 512-byte pieces of head rows.
    wait_vmcnt<0>();
    __syncthreads();  // E1: denominators published, stages free
    float* ob = reinterpret_cast<float*>(&sm.stage[0][0]) + v * (kH * kOPad);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hh = 16 * mb + 4 * q4 + r;
        const float l_run = sm.lsum[0][hh] + sm.lsum[1][hh];
        f[r] = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) ob[(16 * mb + 4 * q4 + r) * kOPad + 16 * nb + l16] = o[mb][nb][r] * f[r];
    }
    float* __restrict__ orow = out + out_row * kH * kDL + 128 * v + 4 * (lane & 31);
#pragma unroll
    for (int j = 0; j < kH / 2; ++j) {
      const int hh = 2 * j + (lane >> 5);
      const f32x4 val = *reinterpret_cast<const f32x4*>(&ob[hh * kOPad + 4 * (lane & 31)]);
      __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(orow + (int64_t)hh * kDL));
    }
  };

  // The query's Q block (64 heads x 576 dims, 72 KB, contiguous) is copied
  // into stages 2-3 by all 8 waves (9 direct-to-LDS loads each) before the
  // census, whose wait covers it; the score waves then take their fragments
  // from LDS. The stages are not loaded before the first tile iteration.
  {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(q) + (int64_t)i * (kH * kRowBytes);
    const uint32_t q_lds = stage0_lds + 2 * kStageBytes;
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const uint32_t chunk = (uint32_t)(8 * c + wave);
      dma16(qb, 1024u * chunk + lane16, q_lds + 1024u * chunk);
    }
  }
  if (wave < 4) {
    census();
    // Q fragments (B operand of the score waves): head 32 g + 16 hb + l16,
    // k-step u covers dims 32u + 8 q4 .. +7.
    bf16x8 qf[2][18];
    const uint32_t q_lds = stage0_lds + 2 * kStageBytes;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const uint32_t qsrc = q_lds + (uint32_t)((32 * (wave & 1) + 16 * hb + l16) * kRowBytes + 16 * q4);
#pragma unroll
      for (int u = 0; u < 18; ++u) qf[hb][u] = __builtin_bit_cast(bf16x8, lds_read16(qsrc + 64 * u));
    }
    if (hilo) score_role(std::true_type{}, qf);
    else score_role(std::false_type{}, qf);
  } else {
    census();
    if (hilo) pv_role(std::true_type{});
    else pv_role(std::false_type{});
  }
}

// Merge of the split partials: for each (query, head), with per-split lse_s
// and normalised outputs o_s, lse = log sum_s exp(lse_s) and
// out = sum_s exp(lse_s - lse) o_s (splits without a valid slot have
// lse_s = -inf and weight 0). One workgroup per (query, head), 4 dims per thread.
constexpr int kCombineThreads = kDL / 4;
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(int n_q, int splits,
                                                                      const float* __restrict__ part_out,
                                                                      const float* __restrict__ part_lse,
                                                                      float* __restrict__ out, float* __restrict__ lse) {
  lds_poison();
  const int i = blockIdx.x, h = blockIdx.y;
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, part_lse[((int64_t)s * n_q + i) * kH + h]);
  f32x4 acc = {0, 0, 0, 0};
  float sum = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float ls = part_lse[((int64_t)s * n_q + i) * kH + h];
      const float wgt = expf(ls - m);  // 0 for an empty split
      sum += wgt;
      if (wgt != 0.0f) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(part_out + (((int64_t)s * n_q + i) * kH + h) * kDL +
                                                        4 * threadIdx.x);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += wgt * o[e];
      }
    }
  }
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] *= inv;
  *reinterpret_cast<f32x4*>(out + ((int64_t)i * kH + h) * kDL + 4 * threadIdx.x) = acc;
  if (lse && threadIdx.x == 0) lse[(int64_t)i * kH + h] = sum > 0.0f ? m + logf(sum) : -INFINITY;
}

hipError_t check_mla_kernels_now() {
  const struct {
    const void* fn;
    int threads;
    size_t dyn_lds;
  } ks[] = {
      {reinterpret_cast<const void*>(mla_mfma_kernel), kThreads, 0},
      {reinterpret_cast<const void*>(mla_combine_kernel), kCombineThreads, 0},
      {reinterpret_cast<const void*>(mla_plain_kernel<uint16_t>), kPlainThreads,
       sizeof(float) * kPlainMlaMaxDqk + (sizeof(float) + sizeof(int32_t)) * kPlainMlaMaxTopk},
      {reinterpret_cast<const void*>(mla_plain_kernel<float>), kPlainThreads,
       sizeof(float) * kPlainMlaMaxDqk + (sizeof(float) + sizeof(int32_t)) * kPlainMlaMaxTopk},
  };
  for (const auto& k : ks) {
    const hipError_t e = check_launch_limits(k.fn, k.threads, k.dyn_lds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t check_mla_kernels() {
  static PerDeviceCache cache;
  return once_per_device(cache, check_mla_kernels_now);
}

hipError_t launch_mla_decode(const MlaArgs& a, void* workspace, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  const MlaSplit sp = mla_decode_split(a);
  if (sp.splits <= 1) return launch_mla(a, s);
  float* part_out = static_cast<float*>(workspace);
  float* part_lse = part_out + (size_t)sp.splits * a.n_q * kH * kDL;
  const float scale_log2 = a.sm_scale * 1.44269504088896340736f;
  hipError_t e = launch_kernel(mla_mfma_kernel, dim3(a.n_q, sp.splits), dim3(kThreads), 0, s, a.n_q, a.offset,
                               a.top_k, sp.split_slots, scale_log2, static_cast<const uint16_t*>(a.q),
                               static_cast<const uint16_t*>(a.kv), a.idx, part_out, part_lse);
  if (e != hipSuccess) return e;
  return launch_kernel(mla_combine_kernel, dim3(a.n_q, kH), dim3(kCombineThreads), 0, s, a.n_q, sp.splits,
                       static_cast<const float*>(part_out), static_cast<const float*>(part_lse), a.out, a.lse);
}

// Library-owned scratch for callers that cannot allocate: the split partials
// of a decode call (kDecodeScratchBytes, one copy per GPU, kept until the
// process ends). Host code never uses this name as an address: the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;  // device id -> that device's copy of `scratch`
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr.emplace(dev, p);
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (mla_fast_path(a)) {
    const float scale_log2 = a.sm_scale * 1.44269504088896340736f;
    return launch_kernel(mla_mfma_kernel, dim3(a.n_q, 1), dim3(kThreads), 0, s, a.n_q, a.offset, a.top_k, a.top_k,
                         scale_log2, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.kv), a.idx,
                         a.out, a.lse);
  }
  const int d_qk = a.d_latent + a.d_rope;
  const size_t lds = sizeof(float) * (size_t)d_qk + (sizeof(float) + sizeof(int32_t)) * (size_t)a.top_k;
  if (a.bf16)
    return launch_kernel(mla_plain_kernel<uint16_t>, dim3(a.n_q, a.n_heads), dim3(kPlainThreads), lds, s, a.offset,
                         a.n_heads, d_qk, a.d_latent, a.top_k, a.sm_scale, static_cast<const uint16_t*>(a.q),
                         static_cast<const uint16_t*>(a.kv), a.idx, a.out, a.lse);
  return launch_kernel(mla_plain_kernel<float>, dim3(a.n_q, a.n_heads), dim3(kPlainThreads), lds, s, a.offset,
                       a.n_heads, d_qk, a.d_latent, a.top_k, a.sm_scale, static_cast<const float*>(a.q),
                       static_cast<const float*>(a.kv), a.idx, a.out, a.lse);
}

}  // namespace dsa
