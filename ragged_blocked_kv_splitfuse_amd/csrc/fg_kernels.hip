// Device side: KV append and ragged blocked attention for gfx950 (MI355X), plus the C-ABI
// entry points that launch them.
//
// Attention is exact softmax attention computed with the online (running max / running sum)
// rescaling of FlashAttention (DeepSpeed-FastGen paper card by Holmes et al. 2024, "Key
// points" and "References" 12-13: FlashAttention-derived kernels), over a PagedAttention-style
// blocked cache (same card, "Key points").  Nothing of those kernels' CUDA design is reused;
// the layout below is built around CDNA4's 64-lane waves and its 16x16x32 bf16 MFMA.
//
// Notation: query row = (new token, query head of the KV head's group); a work record (see
// fg_internal.h) names one sequence, one KV head, a run of query tokens and a key range.
//
// MFMA formulation.  Scores are computed transposed, S^T = K . Q^T, with K as the A operand
// (16 keys x 32 features per instruction) and Q^T as the B operand (32 features x 16 rows).
// The 16x16 result leaves lane l with four keys for query row l%16.  Loading the A operand
// with key rows permuted as 8*(m/4) + 4*a + m%4 (a = which of two 16-key MFMAs) makes lane
// l own eight *consecutive* keys (8*(l/16) .. +7) of a 32-key half tile for its row — exactly
// the B operand layout of the second product O^T = V^T . P^T (k = 32 keys).  P therefore
// never leaves registers, and the A operand V^T needs eight consecutive keys of one feature,
// which the feature-major V block layout provides as one 16-byte load.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fg_internal.h"

using namespace fgi;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

namespace {

constexpr int D = 128;          // head dim of the bf16 kernels
constexpr int KT = KEY_TILE;    // keys per tile
constexpr int NW = 4;           // waves per workgroup
constexpr int NT = NW * 64;     // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 ld16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float *p) {
  uint4 r;
  r.x = bf16_bits(p[0]) | (bf16_bits(p[1]) << 16);
  r.y = bf16_bits(p[2]) | (bf16_bits(p[3]) << 16);
  r.z = bf16_bits(p[4]) | (bf16_bits(p[5]) << 16);
  r.w = bf16_bits(p[6]) | (bf16_bits(p[7]) << 16);
  return as_bf16x8(r);
}

// keep elements i < n of eight packed bf16 values, zero the rest (n in [0, 8])
__device__ __forceinline__ uint4 keep_first(uint4 v, int n) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (2 * i < n) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * i + 1 < n) ? 0xffff0000u : 0u;
    w[i] &= (lo | hi);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

__device__ __forceinline__ int clamp_block(int b, int nb) { return b < 0 ? 0 : (b >= nb ? nb - 1 : b); }

// Swizzles of the LDS tiles (16-byte chunk index XOR a row function) that make the MFMA
// operand reads and the cooperative tile writes free of bank conflicts.
__device__ __forceinline__ int swz_k(int key) { return ((key >> 1) & 12) | (key & 3); }
__device__ __forceinline__ int swz_v(int d) { return (d & 7) ^ ((d >> 3) & 1); }

struct Params {
  const int32_t *work;
  const int32_t *query_start;
  const int32_t *context_len;
  const int32_t *n_query;
  const int32_t *block_table;
  int32_t table_stride;
  int32_t num_tokens;
  const u16 *q;
  const u16 *k_pool;
  const u16 *v_pool;
  u16 *out;
  float *ws;          // workspace as floats (partials)
  int32_t *counters;  // workspace head (split counters)
  int64_t ws_floats;
  int32_t Hq, Hkv, G, bs, bs_log2, num_blocks;
  float sl2;          // scale * log2(e)
};

struct Rec {
  int s, h, tok0, ntok, klo, khi, mode, group, split, nsplit, poff;
};

__device__ __forceinline__ Rec load_rec(const int32_t *w) {
  Rec r;
  r.s = w[W_SEQ];
  r.h = w[W_KVH];
  r.tok0 = w[W_TOK0];
  r.ntok = w[W_NTOK];
  r.klo = w[W_KLO];
  r.khi = w[W_KHI];
  r.mode = w[W_MODE];
  r.group = w[W_GROUP];
  r.split = w[W_SPLIT];
  r.nsplit = w[W_NSPLIT];
  r.poff = w[W_POFF];
  return r;
}

// Final normalisation and bf16 store of 8 consecutive features of one query row.
__device__ __forceinline__ void store_out8(const Params &P, int t, int head, int d0,
                                           const float *o, float inv_l) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = o[i] * inv_l;
  bf16x8 b = pack_bf16x8(v);
  *reinterpret_cast<uint4 *>(P.out + ((size_t)t * P.Hq + head) * D + d0) =
      __builtin_bit_cast(uint4, b);
}

// The last workgroup of a split group merges every split's (m, l, acc) partial in split
// order (so the result does not depend on which workgroup finished last) and writes O.
__device__ void merge_splits(const Params &P, const Rec &R, int rows, int c0_tok, int qs) {
  const int64_t slot = slot_floats(R.mode, D);
  const int cap = R.mode == MODE_STREAM ? STREAM_ROWS : TILE_ROWS;
  for (int idx = threadIdx.x; idx < rows * (D / 8); idx += NT) {
    const int row = idx / (D / 8), chunk = idx % (D / 8);
    float M = NEG_INF;
    for (int k = 0; k < R.nsplit; ++k) {
      const float *sp = P.ws + R.poff + k * slot;
      M = fmaxf(M, sp[cap * D + row]);
    }
    float L = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < R.nsplit; ++k) {
      const float *sp = P.ws + R.poff + k * slot;
      const float m = sp[cap * D + row];
      const float f = (m == NEG_INF) ? 0.f : exp2f(m - M);
      L += sp[cap * D + cap + row] * f;
      const float4 a = *reinterpret_cast<const float4 *>(sp + row * D + chunk * 8);
      const float4 b = *reinterpret_cast<const float4 *>(sp + row * D + chunk * 8 + 4);
      o[0] += a.x * f; o[1] += a.y * f; o[2] += a.z * f; o[3] += a.w * f;
      o[4] += b.x * f; o[5] += b.y * f; o[6] += b.z * f; o[7] += b.w * f;
    }
    const int t = qs + c0_tok + row / P.G;
    const int head = R.h * P.G + row % P.G;
    if (t < P.num_tokens) store_out8(P, t, head, chunk * 8, o, 1.f / L);
  }
}

// Returns true in every thread of the workgroup that must merge the group (the last one).
__device__ bool arrive_last(const Params &P, const Rec &R, int *flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(P.counters + R.group, 1);
    *flag = (prev == R.nsplit - 1);
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

__device__ __forceinline__ void reset_counter(const Params &P, const Rec &R) {
  __syncthreads();
  if (threadIdx.x == 0) atomicExch(P.counters + R.group, 0);
}

// ---------------------------------------------------------------------------------------
// MODE_STREAM: <= 16 query rows.  Each wave streams its own key tiles (w, w+4, ...) straight
// from HBM into MFMA operand registers (no LDS staging, no barriers), then the four waves
// merge their running states through LDS.
// ---------------------------------------------------------------------------------------
__device__ void stream_record(const Params &P, const Rec &R, unsigned char *smem) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const int c = P.context_len[R.s], qs = P.query_start[R.s];
  const int L = c + P.n_query[R.s];
  const int rows = R.ntok * P.G;
  const int32_t *bt = P.block_table + (size_t)R.s * P.table_stride;
  const int bs_mask = P.bs - 1;

  // this lane's query row (r) and its causal limit
  const bool row_ok = r < rows;
  const int row_tok = R.tok0 + r / P.G;
  const int lim = c + row_tok;  // keys 0 .. lim are visible
  bf16x8 qf[D / 32];
  {
    const int t = qs + row_tok, head = R.h * P.G + r % P.G;
    const u16 *qp = P.q + ((size_t)t * P.Hq + head) * D + 8 * g;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
      qf[dc] = (row_ok && t < P.num_tokens) ? as_bf16x8(ld16(qp + 32 * dc)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  float m_run = NEG_INF, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t_begin = R.klo / KT, t_end = (R.khi + KT - 1) / KT;
  const size_t head_stride = (size_t)P.bs * D;  // elements per (block, head) in either pool
  for (int kt = t_begin + w; kt < t_end; kt += NW) {
    const int k0 = kt * KT;
    // ---- K operand: 2 halves x 2 sub-tiles x D/32 chunks, key rows permuted -------------
    bf16x8 kf[2][2][D / 32];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int key = min(k0 + 32 * kh + 8 * (r >> 2) + 4 * a + (r & 3), L - 1);
        const int blk = clamp_block(bt[key >> P.bs_log2], P.num_blocks);
        const u16 *kp = P.k_pool + ((size_t)blk * P.Hkv + R.h) * head_stride +
                        (size_t)(key & bs_mask) * D + 8 * g;
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) kf[kh][a][dc] = as_bf16x8(ld16(kp + 32 * dc));
      }
    // ---- V^T operand: 2 halves x D/16 feature tiles, 8 consecutive keys per lane --------
    uint4 vr[2][D / 16];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int key0 = k0 + 32 * kh + 8 * g;
      const int keyc = min(key0, (L - 1) & ~7);
      const int blk = clamp_block(bt[keyc >> P.bs_log2], P.num_blocks);
      const u16 *vp = P.v_pool + ((size_t)blk * P.Hkv + R.h) * head_stride + (keyc & bs_mask) +
                      (size_t)r * P.bs;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) vr[kh][dt] = ld16(vp + (size_t)16 * dt * P.bs);
      if (k0 + KT > R.khi) {  // keys at or past khi: zero V so stale bits cannot reach O
        const int nvalid = min(max(R.khi - key0, 0), 8);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) vr[kh][dt] = keep_first(vr[kh][dt], nvalid);
      }
    }
    // ---- S^T = K . Q^T ---------------------------------------------------------------
    f32x4 st[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        st[kh][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) st[kh][a] = mfma_bf16(kf[kh][a][dc], qf[dc], st[kh][a]);
      }
    // ---- online softmax (lane holds keys k0 + 32kh + 8g + 4a + j of row r) ---------------
    const bool need_mask = (k0 + KT > R.khi) || (k0 + KT - 1 > c + R.tok0);
    float sv[2][8];
    float tmax = NEG_INF;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k0 + 32 * kh + 8 * g + 4 * a + j;
          float x = st[kh][a][j] * P.sl2;
          if (need_mask && (key > lim || key >= R.khi)) x = NEG_INF;
          sv[kh][4 * a + j] = x;
          tmax = fmaxf(tmax, x);
        }
    tmax = wave_max_xor(tmax, 16);
    tmax = wave_max_xor(tmax, 32);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[kh][i] = exp2f(sv[kh][i] - m_use);
        psum += sv[kh][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
    // ---- O^T += V^T . P^T ------------------------------------------------------------
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const bf16x8 pf = pack_bf16x8(sv[kh]);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma_bf16(as_bf16x8(vr[kh][dt]), pf, acc[dt]);
    }
  }
  // row sum over the four lanes that share row r
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // ---- merge the four waves through LDS ------------------------------------------------
  constexpr int OP = D + 4;  // padded row of the per-wave O^T dump
  float *so = reinterpret_cast<float *>(smem);                 // [NW][16][OP]
  float *sm = so + NW * STREAM_ROWS * OP;                      // [NW][16]
  float *sl = sm + NW * STREAM_ROWS;                           // [NW][16]
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4 *>(so + (w * STREAM_ROWS + r) * OP + 16 * dt + 4 * g) = acc[dt];
  if (g == 0) {
    sm[w * STREAM_ROWS + r] = m_run;
    sl[w * STREAM_ROWS + r] = l_run;
  }
  __syncthreads();
  {
    const int row = threadIdx.x >> 4, chunk = threadIdx.x & 15;  // 16 rows x 16 chunks of 8
    float M = NEG_INF;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm[ww * STREAM_ROWS + row]);
    float Lsum = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float m = sm[ww * STREAM_ROWS + row];
      const float f = (m == NEG_INF) ? 0.f : exp2f(m - M);
      Lsum += sl[ww * STREAM_ROWS + row] * f;
      const float *src = so + (ww * STREAM_ROWS + row) * OP + chunk * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] += src[i] * f;
    }
    if (row < rows) {
      if (R.group < 0) {
        const int t = qs + R.tok0 + row / P.G;
        if (t < P.num_tokens) store_out8(P, t, R.h * P.G + row % P.G, chunk * 8, o, 1.f / Lsum);
      } else {
        float *sp = P.ws + R.poff + (int64_t)R.split * slot_floats(MODE_STREAM, D);
        *reinterpret_cast<float4 *>(sp + row * D + chunk * 8) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4 *>(sp + row * D + chunk * 8 + 4) = make_float4(o[4], o[5], o[6], o[7]);
        if (chunk == 0) {
          sp[STREAM_ROWS * D + row] = M;
          sp[STREAM_ROWS * D + STREAM_ROWS + row] = Lsum;
        }
      }
    }
  }
  if (R.group >= 0) {
    int *flag = reinterpret_cast<int *>(sl + NW * STREAM_ROWS);
    if (arrive_last(P, R, flag)) {
      merge_splits(P, R, rows, R.tok0, qs);
      reset_counter(P, R);
    }
  }
}

// ---------------------------------------------------------------------------------------
// MODE_TILE: up to 128 query rows (chunk rows).  Wave w owns rows [32w, 32w+32) as two
// 16-row MFMA tiles; each 64-key K/V tile is gathered cooperatively (coalesced 16-byte
// loads through the block table) into double-buffered, swizzled LDS and shared by all waves.
// ---------------------------------------------------------------------------------------
constexpr int KTILE_ELEMS = KT * D;   // K tile [64 keys][128]
constexpr int VTILE_ELEMS = D * KT;   // V^T tile [128 features][64 keys]
constexpr int BUF_ELEMS = KTILE_ELEMS + VTILE_ELEMS;

__device__ void tile_record(const Params &P, const Rec &R, unsigned char *smem) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r = lane & 15;
  const int c = P.context_len[R.s], qs = P.query_start[R.s];
  const int L = c + P.n_query[R.s];
  const int rows = R.ntok * P.G;
  const int32_t *bt = P.block_table + (size_t)R.s * P.table_stride;
  const int bs_mask = P.bs - 1;
  const size_t head_stride = (size_t)P.bs * D;
  u16 *lds = reinterpret_cast<u16 *>(smem);

  const int nrt = rows > 32 * w ? (rows > 32 * w + 16 ? 2 : 1) : 0;
  bf16x8 qf[2][D / 32];
  int lim[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = 32 * w + 16 * rt + r;
    const int tok = R.tok0 + row / P.G;
    lim[rt] = c + tok;
    const int t = qs + tok, head = R.h * P.G + row % P.G;
    const bool ok = row < rows && t < P.num_tokens;
    const u16 *qp = P.q + ((size_t)t * P.Hq + head) * D + 8 * g;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
      qf[rt][dc] = ok ? as_bf16x8(ld16(qp + 32 * dc)) : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  float m_run[2] = {NEG_INF, NEG_INF}, l_run[2] = {0.f, 0.f};
  f32x4 acc[2][D / 16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // cooperative tile load: K chunk q -> (key q>>4, 16-byte chunk q&15);
  //                        V chunk q -> (feature q>>3, 8-key chunk q&7)
  uint4 kreg[4], vreg[4];
  auto gload = [&](int kt) {
    const int k0 = kt * KT;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qi = tid + NT * p;
      const int key = min(k0 + (qi >> 4), L - 1);
      const int blk = clamp_block(bt[key >> P.bs_log2], P.num_blocks);
      kreg[p] = ld16(P.k_pool + ((size_t)blk * P.Hkv + R.h) * head_stride +
                     (size_t)(key & bs_mask) * D + 8 * (qi & 15));
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qi = tid + NT * p;
      const int d = qi >> 3;
      const int key0 = k0 + 8 * (qi & 7);
      const int keyc = min(key0, (L - 1) & ~7);
      const int blk = clamp_block(bt[keyc >> P.bs_log2], P.num_blocks);
      uint4 v = ld16(P.v_pool + ((size_t)blk * P.Hkv + R.h) * head_stride + (size_t)d * P.bs +
                     (keyc & bs_mask));
      if (key0 + 8 > R.khi) v = keep_first(v, min(max(R.khi - key0, 0), 8));
      vreg[p] = v;
    }
  };
  auto swrite = [&](int buf) {
    u16 *Kl = lds + buf * BUF_ELEMS;
    u16 *Vl = Kl + KTILE_ELEMS;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qi = tid + NT * p;
      const int key = qi >> 4, ch = qi & 15;
      *reinterpret_cast<uint4 *>(Kl + key * D + 8 * (ch ^ swz_k(key))) = kreg[p];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int qi = tid + NT * p;
      const int d = qi >> 3, ch = qi & 7;
      *reinterpret_cast<uint4 *>(Vl + d * KT + 8 * (ch ^ swz_v(d))) = vreg[p];
    }
  };

  const int t_begin = R.klo / KT, t_end = (R.khi + KT - 1) / KT;
  gload(t_begin);
  swrite(0);
  __syncthreads();
  for (int kt = t_begin; kt < t_end; ++kt) {
    const int buf = (kt - t_begin) & 1;
    const bool more = kt + 1 < t_end;
    if (more) gload(kt + 1);
    if (nrt > 0) {
      const u16 *Kl = lds + buf * BUF_ELEMS;
      const u16 *Vl = Kl + KTILE_ELEMS;
      const int k0 = kt * KT;
      f32x4 st[2][2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int a = 0; a < 2; ++a) st[rt][kh][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int keyl = 32 * kh + 8 * (r >> 2) + 4 * a + (r & 3);
          const u16 *kb = Kl + keyl * D;
          const int sw = swz_k(keyl);
#pragma unroll
          for (int dc = 0; dc < D / 32; ++dc) {
            const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4 *>(kb + 8 * ((4 * dc + g) ^ sw)));
            st[0][kh][a] = mfma_bf16(kf, qf[0][dc], st[0][kh][a]);
            if (nrt > 1) st[1][kh][a] = mfma_bf16(kf, qf[1][dc], st[1][kh][a]);
          }
        }
      const bool need_mask = (k0 + KT > R.khi) || (k0 + KT - 1 > c + R.tok0);
      bf16x8 pf[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if (rt >= nrt) break;
        float sv[2][8];
        float tmax = NEG_INF;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = k0 + 32 * kh + 8 * g + 4 * a + j;
              float x = st[rt][kh][a][j] * P.sl2;
              if (need_mask && (key > lim[rt] || key >= R.khi)) x = NEG_INF;
              sv[kh][4 * a + j] = x;
              tmax = fmaxf(tmax, x);
            }
        tmax = wave_max_xor(tmax, 16);
        tmax = wave_max_xor(tmax, 32);
        const float m_new = fmaxf(m_run[rt], tmax);
        const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
        const float alpha = exp2f(m_run[rt] - m_use);
        float psum = 0.f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            sv[kh][i] = exp2f(sv[kh][i] - m_use);
            psum += sv[kh][i];
          }
        l_run[rt] = l_run[rt] * alpha + psum;
        m_run[rt] = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[rt][dt] *= alpha;
        pf[rt][0] = pack_bf16x8(sv[0]);
        pf[rt][1] = pack_bf16x8(sv[1]);
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int d = 16 * dt + r;
          const bf16x8 vf = as_bf16x8(
              *reinterpret_cast<const uint4 *>(Vl + d * KT + 8 * ((4 * kh + g) ^ swz_v(d))));
          acc[0][dt] = mfma_bf16(vf, pf[0][kh], acc[0][dt]);
          if (nrt > 1) acc[1][dt] = mfma_bf16(vf, pf[1][kh], acc[1][dt]);
        }
    }
    if (more) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------------
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (rt >= nrt) break;
    float l = l_run[rt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = 32 * w + 16 * rt + r;
    if (row >= rows) continue;
    if (R.group < 0) {
      const int t = qs + R.tok0 + row / P.G;
      const int head = R.h * P.G + row % P.G;
      if (t >= P.num_tokens) continue;
      const float inv = 1.f / l;
      u16 *op = P.out + ((size_t)t * P.Hq + head) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const f32x4 a = acc[rt][dt];
        uint2 v;
        v.x = bf16_bits(a[0] * inv) | (bf16_bits(a[1] * inv) << 16);
        v.y = bf16_bits(a[2] * inv) | (bf16_bits(a[3] * inv) << 16);
        *reinterpret_cast<uint2 *>(op + 16 * dt) = v;
      }
    } else {
      float *sp = P.ws + R.poff + (int64_t)R.split * slot_floats(MODE_TILE, D);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        *reinterpret_cast<f32x4 *>(sp + row * D + 16 * dt + 4 * g) = acc[rt][dt];
      if (g == 0) {
        sp[TILE_ROWS * D + row] = m_run[rt];
        sp[TILE_ROWS * D + TILE_ROWS + row] = l;
      }
    }
  }
  if (R.group >= 0) {
    int *flag = reinterpret_cast<int *>(smem);  // tile buffers are no longer needed
    __syncthreads();
    if (arrive_last(P, R, flag)) {
      merge_splits(P, R, rows, R.tok0, qs);
      reset_counter(P, R);
    }
  }
}

constexpr int SMEM_BYTES = 2 * BUF_ELEMS * 2;  // 64 KiB: two K + V^T tile buffers

__global__ __launch_bounds__(NT, 2) void attention_bf16_kernel(Params P) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];
  const Rec R = load_rec(P.work + (size_t)blockIdx.x * FG_WORK_INTS);
  if (R.s < 0 || R.mode < 0) return;
  if (R.group >= 0 &&
      (int64_t)R.poff + (int64_t)R.nsplit * slot_floats(R.mode, D) > P.ws_floats)
    return;  // record inconsistent with the workspace: never write outside it
  if (R.mode == MODE_STREAM)
    stream_record(P, R, smem);
  else
    tile_record(P, R, smem);
}

// ---------------------------------------------------------------------------------------
// fp32 attention: one wave per (token, query head), fp32 FMA throughout.  The accuracy path
// (tiny fp32 workloads); lanes own keys for the scores and features for the output.
// ---------------------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(64) void attention_f32_kernel(
    const int32_t *__restrict__ query_start, const int32_t *__restrict__ context_len,
    const int32_t *__restrict__ block_table, int32_t table_stride, int32_t num_seqs,
    const float *__restrict__ q, const float *__restrict__ k_pool,
    const float *__restrict__ v_pool, float *__restrict__ out, int32_t Hq, int32_t Hkv,
    int32_t bs, int32_t bs_log2, int32_t num_blocks, float scale) {
  __shared__ float sq[HD];
  const int t = blockIdx.x / Hq, gq = blockIdx.x % Hq, lane = threadIdx.x;
  int lo = 0, hi = num_seqs;  // find s with query_start[s] <= t < query_start[s+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (query_start[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int c = context_len[s];
  const int lim = c + (t - query_start[s]);  // keys 0..lim
  const int h = gq / (Hq / Hkv);
  const int32_t *bt = block_table + (size_t)s * table_stride;
  for (int d = lane; d < HD; d += 64) sq[d] = q[((size_t)t * Hq + gq) * HD + d];
  __syncthreads();
  constexpr int PER = HD / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float m_run = NEG_INF, l_run = 0.f;
  for (int k0 = 0; k0 <= lim; k0 += 64) {
    const int key = k0 + lane;
    float sv = NEG_INF;
    if (key <= lim) {
      const int blk = clamp_block(bt[key >> bs_log2], num_blocks);
      const float *kp = k_pool + (((size_t)blk * Hkv + h) * bs + (key & (bs - 1))) * HD;
      float dot = 0.f;
      for (int d = 0; d < HD; ++d) dot = fmaf(sq[d], kp[d], dot);
      sv = dot * scale;
    }
    float mt = sv;
    for (int off = 32; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = expf(m_run - m_new);
    const float p = (key <= lim) ? expf(sv - m_new) : 0.f;
    float ps = p;
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] *= alpha;
    const int nk = min(64, lim + 1 - k0);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j, 64);
      const int kk = k0 + j;
      const int blk = clamp_block(bt[kk >> bs_log2], num_blocks);
      const float *vp = v_pool + ((size_t)blk * Hkv + h) * HD * bs + (kk & (bs - 1));
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(pj, vp[(size_t)(lane + 64 * i) * bs], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) out[((size_t)t * Hq + gq) * HD + lane + 64 * i] = acc[i] / l_run;
}

// ---------------------------------------------------------------------------------------
// KV append: one workgroup per new token.  K rows are copied whole (16-byte chunks); V rows
// are scattered feature by feature into the feature-major V block.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const int32_t *__restrict__ query_start, const int32_t *__restrict__ context_len,
    const int32_t *__restrict__ block_table, int32_t table_stride, int32_t num_seqs,
    const T *__restrict__ k_new, const T *__restrict__ v_new, T *__restrict__ k_pool,
    T *__restrict__ v_pool, int32_t Hkv, int32_t hd, int32_t bs, int32_t bs_log2,
    int32_t num_blocks) {
  const int t = blockIdx.x;
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (query_start[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int pos = context_len[s] + (t - query_start[s]);
  const int blk = block_table[(size_t)s * table_stride + (pos >> bs_log2)];
  if (blk < 0 || blk >= num_blocks) return;  // validated on the host; never write out of range
  const int slot = pos & (bs - 1);
  const int row = Hkv * hd;
  // K: Hkv rows of hd elements, each contiguous at (blk, h, slot)
  constexpr int V16 = 16 / sizeof(T);
  const int chunks_per_head = hd / V16;
  for (int i = threadIdx.x; i < Hkv * chunks_per_head; i += blockDim.x) {
    const int h = i / chunks_per_head, ch = i % chunks_per_head;
    const uint4 v = *reinterpret_cast<const uint4 *>(k_new + (size_t)t * row + h * hd + ch * V16);
    *reinterpret_cast<uint4 *>(k_pool + (((size_t)blk * Hkv + h) * bs + slot) * hd + ch * V16) = v;
  }
  // V: element (h, d) goes to ((blk*Hkv + h)*hd + d)*bs + slot
  for (int i = threadIdx.x; i < row; i += blockDim.x) {
    const int h = i / hd, d = i % hd;
    v_pool[(((size_t)blk * Hkv + h) * hd + d) * bs + slot] = v_new[(size_t)t * row + i];
  }
}

}  // namespace

// =======================================================================================
// C ABI
// =======================================================================================
extern "C" {

fg_status fg_kv_append(const fg_cache *cache, const fg_ragged_batch *dev, const void *k_new,
                       const void *v_new, void *stream) {
  clear_error();
  if (!cache || !dev) return fail(FG_E_ARG, "null cache or batch");
  if (dev->num_tokens < 0 || dev->num_seqs < 0) return fail(FG_E_ARG, "negative sizes");
  if (dev->num_tokens == 0) return FG_OK;
  if (dev->num_seqs < 1 || !dev->query_start || !dev->context_len || !dev->block_table)
    return fail(FG_E_ARG, "descriptor arrays are null");
  if (!k_new || !v_new || !cache->k_pool || !cache->v_pool)
    return fail(FG_E_ARG, "k_new, v_new and both pools must be device pointers");
  const fg_cache_config &c = cache->cfg;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(dev->num_tokens), block(256);
  if (c.dtype == FG_BF16) {
    hipLaunchKernelGGL(kv_append_kernel<u16>, grid, block, 0, st, dev->query_start,
                       dev->context_len, dev->block_table, dev->table_stride, dev->num_seqs,
                       (const u16 *)k_new, (const u16 *)v_new, (u16 *)cache->k_pool,
                       (u16 *)cache->v_pool, c.num_kv_heads, c.head_dim, c.block_size,
                       cache->bs_log2, c.num_blocks);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, block, 0, st, dev->query_start,
                       dev->context_len, dev->block_table, dev->table_stride, dev->num_seqs,
                       (const float *)k_new, (const float *)v_new, (float *)cache->k_pool,
                       (float *)cache->v_pool, c.num_kv_heads, c.head_dim, c.block_size,
                       cache->bs_log2, c.num_blocks);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_E_HIP, "kv_append launch: %s", hipGetErrorString(e));
  return FG_OK;
}

fg_status fg_ragged_attention(const fg_cache *cache, const fg_ragged_batch *dev,
                              const fg_attention_plan_info *plan, const int32_t *work_dev,
                              const void *q, int32_t num_q_heads, float scale, void *out,
                              void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  if (!cache || !dev) return fail(FG_E_ARG, "null cache or batch");
  const fg_cache_config &c = cache->cfg;
  if (num_q_heads < 1 || num_q_heads % c.num_kv_heads)
    return fail(FG_E_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                c.num_kv_heads);
  if (dev->num_tokens < 0 || dev->num_seqs < 0) return fail(FG_E_ARG, "negative sizes");
  if (dev->num_tokens == 0) return FG_OK;
  if (dev->num_seqs < 1 || !dev->query_start || !dev->context_len || !dev->block_table ||
      !dev->n_query)
    return fail(FG_E_ARG, "descriptor arrays are null");
  if (!q || !out || !cache->k_pool || !cache->v_pool)
    return fail(FG_E_ARG, "q, out and both pools must be device pointers");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (c.dtype == FG_F32) {
    const dim3 grid((unsigned)dev->num_tokens * num_q_heads), block(64);
    if (c.head_dim == 64)
      hipLaunchKernelGGL(attention_f32_kernel<64>, grid, block, 0, st, dev->query_start,
                         dev->context_len, dev->block_table, dev->table_stride, dev->num_seqs,
                         (const float *)q, (const float *)cache->k_pool,
                         (const float *)cache->v_pool, (float *)out, num_q_heads,
                         c.num_kv_heads, c.block_size, cache->bs_log2, c.num_blocks, scale);
    else
      hipLaunchKernelGGL(attention_f32_kernel<128>, grid, block, 0, st, dev->query_start,
                         dev->context_len, dev->block_table, dev->table_stride, dev->num_seqs,
                         (const float *)q, (const float *)cache->k_pool,
                         (const float *)cache->v_pool, (float *)out, num_q_heads,
                         c.num_kv_heads, c.block_size, cache->bs_log2, c.num_blocks, scale);
  } else {
    if (!plan) return fail(FG_E_ARG, "bf16 attention needs the plan info");
    if (plan->num_q_heads != num_q_heads || plan->num_tokens != dev->num_tokens)
      return fail(FG_E_ARG, "plan was made for another batch (Hq %d, T %d)", plan->num_q_heads,
                  plan->num_tokens);
    if (plan->num_work < 1 || !work_dev) return fail(FG_E_ARG, "empty or null work list");
    if (plan->workspace_bytes > 0 && (!workspace || workspace_bytes < (size_t)plan->workspace_bytes))
      return fail(FG_E_WORKSPACE, "workspace of %zu bytes, plan needs %lld", workspace_bytes,
                  (long long)plan->workspace_bytes);
    if (c.head_dim != D) return fail(FG_E_UNSUPPORTED, "bf16 head_dim %d", c.head_dim);
    if (c.block_size < 8)
      return fail(FG_E_UNSUPPORTED, "bf16 attention reads 8-key runs: block_size %d < 8",
                  c.block_size);
    Params P;
    P.work = work_dev;
    P.query_start = dev->query_start;
    P.context_len = dev->context_len;
    P.n_query = dev->n_query;
    P.block_table = dev->block_table;
    P.table_stride = dev->table_stride;
    P.num_tokens = dev->num_tokens;
    P.q = (const u16 *)q;
    P.k_pool = (const u16 *)cache->k_pool;
    P.v_pool = (const u16 *)cache->v_pool;
    P.out = (u16 *)out;
    P.ws = (float *)workspace;
    P.counters = (int32_t *)workspace;
    P.ws_floats = (int64_t)(workspace ? workspace_bytes / 4 : 0);
    P.Hq = num_q_heads;
    P.Hkv = c.num_kv_heads;
    P.G = num_q_heads / c.num_kv_heads;
    P.bs = c.block_size;
    P.bs_log2 = cache->bs_log2;
    P.num_blocks = c.num_blocks;
    P.sl2 = scale * LOG2E;
    hipLaunchKernelGGL(attention_bf16_kernel, dim3(plan->num_work), dim3(NT), 0, st, P);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_E_HIP, "attention launch: %s", hipGetErrorString(e));
  return FG_OK;
}

}  // extern "C"
