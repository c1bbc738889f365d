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
constexpr int kKRowBytes = kDQK * 2;            // 1152: key-major row (72 x 16-byte pieces)
constexpr int kKBufBytes = kTile * kKRowBytes;  // 36 KB
constexpr int kVtBufBytes = kDL * kTile * 2;    // 32 KB: 512 dim-rows x 32 keys
constexpr int kPBufBytes = kH * kTile * 2;      // 4 KB
constexpr int kHiloMaxValid = 512;  // queries with at most this many valid keys use hi/lo P

struct MlaSmem {
  uint8_t kbuf[kKBufBytes];        // key-major tile, 16-byte pieces XOR-swizzled by row
  uint8_t vtbuf[2][kVtBufBytes];   // dim-major tile (double-buffered)
  uint8_t pbuf[2][kPBufBytes];     // P as bf16 [head][slot]: hi part, lo part
  float alpha[kH];                 // per-head rescale of the running output
  float fin[kH];                   // per-head 1 / l at the end
  union {
    uint32_t vbits;                // validity bit per slot of the staged tile
    uint8_t vbyte[4];              // byte g: slots 8g..8g+7 (written by wave g)
  };
  int last_slot;                   // one past the last valid slot
  int n_valid;
};

// Key-major piece s (0..71) of tile row r lives at piece s ^ (r & 7): a wave
// reading one 16-byte piece of 16 rows, or 64 pieces of one row, touches every
// LDS bank equally.
__device__ __forceinline__ int kpiece_off(int r, int s) { return r * kKRowBytes + 16 * (s ^ (r & 7)); }

// Dim d of the value tile lives in row (d % 8) * 64 + d / 8; its 32 keys form
// 4 pieces of 8 keys, piece g stored at g ^ ((row >> 1) & 3). Both the
// transposing writes (64 lanes -> 64 consecutive rows) and the MFMA operand
// reads (16 dims x 4 pieces) then spread evenly over the banks.
__device__ __forceinline__ int vrow(int d) { return (d & 7) * 64 + (d >> 3); }
__device__ __forceinline__ int vpiece_off(int row, int g) { return row * 64 + 16 * (g ^ ((row >> 1) & 3)); }

__device__ __forceinline__ bool slot_valid(int32_t j, int64_t p) { return j >= 0 && (int64_t)j <= p; }

// Registers one tile ahead: 8 value pieces (keys 8g..8g+7, dims 8c..8c+7) and
// one rope piece (key rk, dims 512 + 8 rc .. +7).
struct Gathered {
  u32x4 v[8];
  u32x4 r;
  uint32_t vmask;  // bit e = key 8g + e valid
  bool rvalid;
};

__device__ __forceinline__ void gather_issue(Gathered& G, const uint16_t* __restrict__ kv,
                                             const int32_t* __restrict__ idx_row, int top_k, int tile,
                                             int64_t p, int g, int c, int rk, int rc) {
  G.vmask = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int slot = tile * kTile + 8 * g + e;
    const int32_t j = slot < top_k ? idx_row[slot] : -1;
    const bool ok = slot_valid(j, p);
    G.vmask |= (uint32_t)ok << e;
    G.v[e] = ok ? *reinterpret_cast<const u32x4*>(kv + (int64_t)j * kDQK + 8 * c) : u32x4{0, 0, 0, 0};
  }
  const int rslot = tile * kTile + rk;
  const int32_t rj = rslot < top_k ? idx_row[rslot] : -1;
  G.rvalid = slot_valid(rj, p);
  G.r = G.rvalid ? *reinterpret_cast<const u32x4*>(kv + (int64_t)rj * kDQK + kDL + 8 * rc) : u32x4{0, 0, 0, 0};
}

__device__ __forceinline__ void gather_commit(const Gathered& G, MlaSmem& sm, int vt, int g, int c, int rk,
                                              int rc, int lane) {
  // key-major copy
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(sm.kbuf + kpiece_off(8 * g + e, c)) = G.v[e];
  *reinterpret_cast<u32x4*>(sm.kbuf + kpiece_off(rk, 64 + rc)) = G.r;
  // transposed copy: for dim 8c + x, the 8 keys 8g..8g+7
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    u32x4 t;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = G.v[2 * w][x >> 1], b = G.v[2 * w + 1][x >> 1];
      t[w] = (x & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
    const int row = vrow(8 * c + x);
    *reinterpret_cast<u32x4*>(sm.vtbuf[vt] + vpiece_off(row, g)) = t;
  }
  if (lane == 0) sm.vbyte[g] = (uint8_t)G.vmask;
}

__global__ __launch_bounds__(kThreads, 1) void mla_mfma_kernel(int n_q, int offset, int top_k, float scale_log2,
                                                               const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ kv,
                                                               const int32_t* __restrict__ idx,
                                                               float* __restrict__ out, float* __restrict__ lse) {
  __shared__ MlaSmem sm;
  const int i = blockIdx.x;
  const int64_t p = (int64_t)offset + i;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int32_t* __restrict__ idx_row = idx + (int64_t)i * top_k;

  // Valid-slot census: early stop after the last valid slot; hi/lo P for few keys.
  if (tid == 0) {
    sm.last_slot = 0;
    sm.n_valid = 0;
  }
  __syncthreads();
  {
    int last = 0, cnt = 0;
    for (int t = tid; t < top_k; t += kThreads) {
      if (slot_valid(idx_row[t], p)) {
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
    for (int ks = 0; ks < kDQK / 32; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qsrc + 32 * ks));
  }
  __syncthreads();
  const int n_tiles = (sm.last_slot + kTile - 1) / kTile;
  const bool hilo = sm.n_valid <= kHiloMaxValid;

  // Gather roles.
  const int g = wave, c = lane;            // value pieces: keys 8g..8g+7, dims 8c..8c+7
  const int rk = tid >> 3, rc = tid & 7;   // rope piece: key rk, dims 512 + 8rc..

  f32x4 o[4][8];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[mb][nb] = f32x4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;  // for head 16*wave + l16

  Gathered G;
  if (n_tiles > 0) {
    gather_issue(G, kv, idx_row, top_k, 0, p, g, c, rk, rc);
    gather_commit(G, sm, 0, g, c, rk, rc, lane);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int vt = t & 1;
    if (t + 1 < n_tiles) gather_issue(G, kv, idx_row, top_k, t + 1, p, g, c, rk, rc);

    // ---- S^T = K Q^T for this wave's 16 heads: two 16-slot blocks.
    f32x4 s[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
    for (int ks = 0; ks < kDQK / 32; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sm.kbuf + kpiece_off(16 * mb + l16, 4 * ks + q4)));
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[mb], 0, 0, 0);
      }
    }
    // ---- online softmax for head 16*wave + l16 over slots 16mb + 4q4 + r.
    const uint32_t vb = sm.vbits;
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 16 * mb + 4 * q4 + r;
        const float v = ((vb >> slot) & 1u) ? s[mb][r] * scale_log2 : -INFINITY;
        s[mb][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = (m_run == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.0f;
    uint32_t phi[2][2], plo[2][2];
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
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    {
      const int head = 16 * wave + l16;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int off = head * (kTile * 2) + 2 * (16 * mb + 4 * q4);
        *reinterpret_cast<u32x2*>(sm.pbuf[0] + off) = u32x2{phi[mb][0], phi[mb][1]};
        if (hilo) *reinterpret_cast<u32x2*>(sm.pbuf[1] + off) = u32x2{plo[mb][0], plo[mb][1]};
      }
      if (q4 == 0) sm.alpha[head] = alpha;
    }
    __syncthreads();

    // ---- O[64 heads][dims 128w..] = alpha * O + P V.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 al = *reinterpret_cast<const f32x4*>(&sm.alpha[16 * mb + 4 * q4]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[mb][nb] *= al;
    }
    {
      bf16x8 pa[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        pa[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sm.pbuf[0] + (16 * mb + l16) * (kTile * 2) + 16 * q4));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int row = vrow(128 * wave + 16 * nb + l16);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sm.vtbuf[vt] + vpiece_off(row, q4)));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mb], vf, o[mb][nb], 0, 0, 0);
      }
      if (hilo) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          pa[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sm.pbuf[1] + (16 * mb + l16) * (kTile * 2) + 16 * q4));
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int row = vrow(128 * wave + 16 * nb + l16);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sm.vtbuf[vt] + vpiece_off(row, q4)));
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) o[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mb], vf, o[mb][nb], 0, 0, 0);
        }
      }
    }
    // ---- stage the next tile (its loads were issued before Q K^T).
    // kbuf and vbits were last read before the barrier above; the other value
    // buffer was last read in the previous tile's P V.
    if (t + 1 < n_tiles) gather_commit(G, sm, vt ^ 1, g, c, rk, rc, lane);
    __syncthreads();
  }

  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2.
  if (q4 == 0) {
    const int head = 16 * wave + l16;
    sm.fin[head] = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
    if (lse) lse[(int64_t)i * kH + head] = (l_run > 0.0f) ? (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f : -INFINITY;
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

bool mla_fast_path(const MlaArgs& a) { return a.bf16 && a.n_heads == kH && a.d_latent == kDL && a.d_rope == kDR; }

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
