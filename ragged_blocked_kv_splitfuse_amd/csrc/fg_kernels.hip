// Device side: KV append and ragged blocked attention for gfx950 (MI355X), plus the C-ABI
// entry points that launch them.
//
// Attention is exact softmax attention computed with the online (running max / running sum)
// rescaling of FlashAttention (DeepSpeed-FastGen paper card by Holmes et al. 2024, "Key
// points" and "References" 12-13: FlashAttention-derived kernels), over a PagedAttention-style
// blocked cache (same card, "Key points").  Nothing of those kernels' CUDA design is reused;
// the layout below is built around CDNA4's 64-lane waves and its 16x16x32 (decode rows) and
// 32x32x16 (chunk rows) bf16 MFMAs.
//
// Notation: query row = (new token, query head of the KV head's group); a work record (see
// fg_internal.h) names one sequence, one KV head, a run of query tokens and a key range.
//
// MFMA formulation (decode rows; the chunk-row variant with 32x32x16 is described at the tile
// path).  Scores are computed transposed, S^T = K . Q^T, with K as the A operand
// (16 keys x 32 features per instruction) and Q^T as the B operand (32 features x 16 rows).
// The 16x16 result leaves lane l with four keys for query row l%16.  Loading the A operand
// with key rows permuted as 8*(m/4) + 4*a + m%4 (a = which of two 16-key MFMAs) makes lane
// l own eight *consecutive* keys (8*(l/16) .. +7) of a 32-key half tile for its row — exactly
// the B operand layout of the second product O^T = V^T . P^T (k = 32 keys).  P therefore
// never leaves registers, and the A operand V^T needs eight consecutive keys of one feature,
// which the V pool layout (keys in groups of 8, each group feature-major with its 8 keys
// adjacent) provides as one 16-byte load.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "fg_internal.h"

using namespace fgi;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

namespace {

// HD (template parameter): head dim of the bf16 kernels, 64 or 128
constexpr int KT = KEY_TILE;    // keys per tile
constexpr int NW = WAVES_PER_WG;  // waves per workgroup
constexpr int NT = NW * 64;     // threads per workgroup
// The LDS stage ring of tile records (also the stream records' merge space)
constexpr int KS = 32;                     // keys per stage
constexpr int NSTAGE = 4;                  // ring depth
constexpr int stage_k(int hd) { return KS * hd; }          // u16 elements of a stage's K part
constexpr int stage_elems(int hd) { return 2 * KS * hd; }  // K + V^T: 16 KiB at HD 128
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 ld16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// the same with the non-temporal hint (data read once: L2 lines it fills are the first evicted)
__device__ __forceinline__ uint4 ld16_nt(const void *p) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v t = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// eight fp32 values -> eight bf16 (hardware round-to-nearest-even conversion)
__device__ __forceinline__ bf16x8 to_bf16x8(const float *p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
  return r;
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over the four lanes l, l^16, l^32, l^48 (the lanes that hold one query row in the
// 16x16 MFMA result layout), with the gfx950 lane-swap instructions instead of LDS permutes.
// v_permlane16_swap applied to two copies of x leaves {x[l], x[l^16]} in the two registers of
// every lane (16-lane rows 0<->1 and 2<->3 trade places); v_permlane32_swap does the same for
// l^32.  Written as one asm block: through the builtins the compiler treated the swap of two
// equal values as a no-op and dropped the max that follows.  The s_nop gives the swap the two
// wait states it needs after a VALU write of its operands.
__device__ __forceinline__ float row_max4(float x) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(t));
  return x;
}

// Max over lanes l and l^32 (the two lanes that hold one query row in the 32x32 MFMA result
// layout): the second half of row_max4.
__device__ __forceinline__ float pair_max(float x) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(t));
  return x;
}

// The running max used for the exponentials is only moved when a row's new max exceeds it
// by more than LAZY_TAU (log2 units).  Softmax does not depend on the shift, so this is exact
// in exact arithmetic; it bounds p by 2^LAZY_TAU and spares the accumulator rescale on most
// key tiles.
constexpr float LAZY_TAU = 8.f;

__device__ __forceinline__ int clamp_block(int b, int nb) { return b < 0 ? 0 : (b >= nb ? nb - 1 : b); }

// Descriptors, block tables and work records are read-only while a kernel runs.  Reading them
// through the constant address space lets wave-uniform reads become scalar loads, which are
// counted apart from the vector loads still in flight (a vector read of a block id would make
// its wait drain every outstanding tile load as well).
typedef __attribute__((address_space(4))) const int32_t cint32_t;
__device__ __forceinline__ int ldc(const int32_t *p, size_t i) {
  return ((cint32_t *)p)[i];
}

struct Params {
  const int32_t *items;  // work items, FG_ITEM_INTS each
  const int32_t *codes;  // record codes: item * Hkv + KV head, -1 for padding
  int32_t num_items;
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
  float *ws;          // workspace as floats (split partials)
  int64_t ws_floats;
  int32_t Hq, Hkv, G, bs, bs_log2, num_blocks;
  float sl2;          // scale * log2(e)
};

struct Rec {
  int s, h, tok0, ntok, klo, khi, mode, group, split, nsplit, poff;
};

// Record `idx`: its code names an item and a KV head.  A padding code, or one naming an item
// outside the list, gives a record with s = -1 (the workgroup exits).
template <int HD>
__device__ __forceinline__ Rec load_rec(const Params &P, int idx) {
  Rec r;
  const int code = ldc(P.codes, idx);
  const int item = code >= 0 ? code / P.Hkv : -1;
  if (item < 0 || item >= P.num_items) {
    r.s = -1;
    r.group = -1;
    return r;
  }
  const int32_t *w = P.items + (size_t)item * FG_ITEM_INTS;
  r.h = code - item * P.Hkv;
  r.s = ldc(w, I_SEQ);
  r.tok0 = ldc(w, I_TOK0);
  r.ntok = ldc(w, I_NTOK);
  r.klo = ldc(w, I_KLO);
  r.khi = ldc(w, I_KHI);
  r.mode = ldc(w, I_MODE);
  r.split = ldc(w, I_SPLIT);
  r.nsplit = ldc(w, I_NSPLIT);
  const int g0 = ldc(w, I_GROUP);
  r.group = g0 >= 0 ? g0 + r.h : -1;
  r.poff = g0 >= 0 ? ldc(w, I_POFF) + r.h * r.nsplit * (int)slot_floats(r.mode, HD) : 0;
  return r;
}

template <int HD>
__device__ __forceinline__ bool rec_fits_workspace(const Params &P, const Rec &R) {
  return R.group < 0 ||
         (int64_t)R.poff + (int64_t)R.nsplit * slot_floats(R.mode, HD) <= P.ws_floats;
}

// Final normalisation and bf16 store of 8 consecutive features of one query row.
template <int HD>
__device__ __forceinline__ void store_out8(const Params &P, int t, int head, int d0,
                                           const float *o, float inv_l) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = o[i] * inv_l;
  *reinterpret_cast<bf16x8 *>(P.out + ((size_t)t * P.Hq + head) * HD + d0) = to_bf16x8(v);
}

// Online softmax over one 64-key tile for one 16-row MFMA tile (FlashAttention's running
// max / running sum).  s[kh][a][j] holds the raw score of key key0 + 32kh + 4a + j for this
// lane's row (key0 = k0 + 8g).  The running max m lives in the scaled log2 domain; p =
// 2^(s*scale*log2e - m).  Updates m, l (this lane's partial row sum), rescales acc when a
// row's max moved, and returns P packed to bf16 as the B operands of the P.V product.
template <int HD>
__device__ __forceinline__ void online_softmax(f32x4 (&s)[2][2], bool need_mask, int key0,
                                               int lim, int khi, float sl2, float &m, float &l,
                                               f32x4 *acc, bf16x8 (&pf)[2]) {
  if (need_mask) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key0 + 32 * kh + 4 * a + j;
          if (key > lim || key >= khi) s[kh][a][j] = NEG_INF;
        }
  }
  float mx = NEG_INF;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[kh][a][j]);
  mx = row_max4(mx) * sl2;
  const bool upd = mx > m + LAZY_TAU;
  const float m_new = upd ? mx : m;
  const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
  const float alpha = fast_exp2(m - m_use);
  float psum = 0.f;
  float p[2][8];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = fast_exp2(fmaf(s[kh][a][j], sl2, -m_use));
        p[kh][4 * a + j] = e;
        psum += e;
      }
  l = l * alpha + psum;
  m = m_new;
  if (__ballot(upd)) {
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) acc[dt] *= alpha;
  }
  pf[0] = to_bf16x8(p[0]);
  pf[1] = to_bf16x8(p[1]);
}

constexpr int merge_rows(int hd) { return NT / (hd / 8); }  // rows one merge workgroup covers

// Combine: the merge record of a split group reads every split's (m, l, acc) partial in
// split order (deterministic) and writes O.  Runs in its own launch after the main kernel.
// Each workgroup merges one MERGE_ROWS-row slice (blockIdx.y) of the group: one thread per (row,
// 8-feature chunk).  The partials of up to MERGE_BATCH splits are requested together, so a
// group costs about one memory latency per batch rather than one per split; the sums still
// run in split order.
constexpr int MERGE_BATCH = 4;

template <int HD>
__device__ void merge_splits(const Params &P, const Rec &R) {
  constexpr int D = HD;
  constexpr int MERGE_ROWS = merge_rows(HD);
  constexpr int KB = MERGE_BATCH;
  const int64_t slot = slot_floats(R.mode, D);
  const int cap = R.mode == MODE_STREAM ? STREAM_ROWS : TILE_ROWS;
  const int rows = R.ntok * P.G;
  const int qs = ldc(P.query_start, R.s);
  const int row = MERGE_ROWS * blockIdx.y + threadIdx.x / (D / 8), chunk = threadIdx.x % (D / 8);
  if (row >= rows) return;
  const float *base = P.ws + R.poff;
  const int ns = R.nsplit;
  float M = NEG_INF;
  for (int k0 = 0; k0 < ns; k0 += KB) {
    float mv[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j)
      mv[j] = (k0 + j < ns) ? base[(int64_t)(k0 + j) * slot + cap * D + row] : NEG_INF;
#pragma unroll
    for (int j = 0; j < KB; ++j) M = fmaxf(M, mv[j]);
  }
  float L = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int k0 = 0; k0 < ns; k0 += KB) {
    float mv[KB], lv[KB];
    float4 av[KB], bv[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (k0 + j < ns) {
        const float *sp = base + (int64_t)(k0 + j) * slot;
        mv[j] = sp[cap * D + row];
        lv[j] = sp[cap * D + cap + row];
        av[j] = *reinterpret_cast<const float4 *>(sp + row * D + chunk * 8);
        bv[j] = *reinterpret_cast<const float4 *>(sp + row * D + chunk * 8 + 4);
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (k0 + j < ns) {
        const float f = (mv[j] == NEG_INF) ? 0.f : fast_exp2(mv[j] - M);
        L += lv[j] * f;
        o[0] += av[j].x * f; o[1] += av[j].y * f; o[2] += av[j].z * f; o[3] += av[j].w * f;
        o[4] += bv[j].x * f; o[5] += bv[j].y * f; o[6] += bv[j].z * f; o[7] += bv[j].w * f;
      }
    }
  }
  const int t = qs + R.tok0 + row / P.G;
  const int head = R.h * P.G + row % P.G;
  if (t < P.num_tokens) store_out8<HD>(P, t, head, chunk * 8, o, 1.f / L);
}

// One wave instruction: 16 bytes per lane from global memory to LDS at lds_wave_base + 16*lane.
// Written as inline asm so that the compiler does not track these loads: its alias tracking of
// LDS-DMA targets is easily lost and then drains every prefetched stage before ordinary LDS
// reads.  The LDS base goes in through an "{m0}" operand, so the compiler itself writes M0 and
// knows it is in use.  The kernel waits for the loads itself (wait_dma) and separates them from
// LDS reads by barriers; the "memory" clobber keeps the compiler from moving memory operations
// across them.
__device__ __forceinline__ void dma16(const u16 *src, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(lds_addr)
               : "memory");
}

// the same with the non-temporal hint, for data read once
__device__ __forceinline__ void dma16_nt(const u16 *src, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "{m0}"(lds_addr)
               : "memory");
}

// LDS byte address of a workgroup-shared array (a constant once the array is known)
__device__ __forceinline__ uint32_t lds_addr_of(const u16 *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const u16 *)p;
}

// Workgroup barrier for the stage ring.  __syncthreads() would also drain every vector load
// still in flight (its fence waits for all of them), i.e. the prefetched stages; here the
// data a stage needs is already covered by wait_dma, and LDS reads complete before their
// MFMAs consume them, so a bare barrier suffices.  The empty asm statements keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until at most n of this wave's LDS-DMA loads are outstanding (n in 0 .. 16)
template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt encoding (gfx9): vmcnt = bits 3:0 (+ bits 15:14), expcnt 6:4, lgkmcnt 11:8
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}
__device__ __forceinline__ void wait_dma(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;   case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;   case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;   case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;   case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;   case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break; case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break; case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break; case 15: wait_vm<15>(); break;
    default: wait_vm<16>(); break;
  }
}

// Stream records stage each 64-key tile's K rows in the wave's own LDS region.  Loaded straight
// into MFMA operand registers, one instruction reads the same 64-byte quarter of 16 key rows, i.e.
// half of 16 cache lines; a CU then moves about a third of what it moves for whole lines (probe:
// 37 against 116 GB/s per CU with the chip otherwise idle).  The LDS-DMA instead fetches whole
// rows (RPI rows of 2*HD bytes per instruction), and the operand reads come from LDS.  With
// every request a whole line, the stream's K and V loads carry the non-temporal hint: a decode
// row's history is read once, and its lines no longer push the chunk rows' K/V out of L2 (with
// half-line requests the hint made the second half miss).  Chunk c of
// key row `key` sits at slot c ^ swz_s<HD>(key): the 16 rows of one operand read (key bits 0, 1,
// 3, 4 vary; bit 2 and 5 are fixed) then fall on 16 distinct 16-byte slots of the bank window (at
// HD 64 two rows share a window: the row's parity picks the half, the swizzle takes 8 values).
template <int HD>
struct StreamK {
  static constexpr int CPR = HD / 8;         // 16-byte chunks per key row
  static constexpr int RPI = 64 / CPR;       // key rows per DMA instruction (1 KiB)
  static constexpr int NDMA = KEY_TILE / RPI;  // DMA instructions per tile
  static constexpr int ELEMS = KEY_TILE * HD;  // u16 elements of a wave's region
};
template <int HD>
__device__ __forceinline__ int swz_s(int key) {
  if (HD == 128) return ((key >> 1) & 12) | (key & 3);
  return ((key >> 1) & 1) | ((key >> 2) & 6);
}

// ---------------------------------------------------------------------------------------
// MODE_STREAM: <= 16 query rows.  Each wave streams its own key tiles (w, w + NW, ...) from
// HBM: V straight into MFMA operand registers, K (where a tile lies in one block) through the
// wave's own LDS region in whole rows; no barriers until the NW waves merge their running
// states through LDS.
// ---------------------------------------------------------------------------------------
template <int HD, bool BIG, typename LdsT>
__device__ void stream_record(const Params &P, const Rec &R, const LdsT &S) {
  constexpr int D = HD;
  constexpr int STAGE_K = stage_k(HD);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const int c = ldc(P.context_len, R.s), qs = ldc(P.query_start, R.s);
  const int L = c + ldc(P.n_query, R.s);
  const int rows = R.ntok * P.G;
  const int32_t *bt = P.block_table + (size_t)R.s * P.table_stride;
  const int bs_mask = P.bs - 1;
  const size_t head_stride = (size_t)P.bs * D;  // elements per (block, head) in either pool

  using SK = StreamK<HD>;
  const u16 *kw = S.base + w * SK::ELEMS;  // this wave's K region
  const uint32_t kw_lds = __builtin_amdgcn_readfirstlane(lds_addr_of(kw));  // wave-uniform
  const bool row_ok = r < rows;
  const int row_tok = R.tok0 + r / P.G;
  const int lim = c + row_tok;  // keys 0 .. lim are visible to this lane's row
  bf16x8 qf[D / 32];
  {
    const int t = qs + row_tok, head = R.h * P.G + r % P.G;
    const u16 *qp = P.q + ((size_t)t * P.Hq + head) * D + 8 * g;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
      qf[dc] = (row_ok && t < P.num_tokens) ? as_bf16x8(ld16(qp + 32 * dc))
                                           : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  float m_run = NEG_INF, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t_begin = R.klo / KT, t_end = (R.khi + KT - 1) / KT;
  // Block ids are read one tile ahead (raw, clamped where used), so that a tile's K/V loads
  // never wait behind a fresh block-table read: the two latencies would add up per tile.
  // BIG: one scalar id per tile; otherwise per lane, for its four K rows and two V runs.
  auto k_key = [&](int k0, int kh, int a) {
    return min(k0 + 32 * kh + 8 * (r >> 2) + 4 * a + (r & 3), L - 1);
  };
  auto v_key = [&](int k0, int kh) { return min(k0 + 32 * kh + 8 * g, (L - 1) & ~7); };
  int id_t = 0, id_k[2][2] = {{0, 0}, {0, 0}}, id_v[2] = {0, 0};
  auto read_ids = [&](int kt) {
    const int k0 = kt * KT;
    if (BIG) {
      id_t = ldc(bt, k0 >> P.bs_log2);
    } else {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int a = 0; a < 2; ++a) id_k[kh][a] = bt[k_key(k0, kh, a) >> P.bs_log2];
        id_v[kh] = bt[v_key(k0, kh) >> P.bs_log2];
      }
    }
  };
  if (t_begin + w < t_end) read_ids(t_begin + w);
  for (int kt = t_begin + w; kt < t_end; kt += NW) {
    const int k0 = kt * KT;
    const int blk_t = BIG ? clamp_block(id_t, P.num_blocks) : 0;
    int blk_k[2][2], blk_v[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int a = 0; a < 2; ++a) blk_k[kh][a] = clamp_block(id_k[kh][a], P.num_blocks);
      blk_v[kh] = clamp_block(id_v[kh], P.num_blocks);
    }
    if (kt + NW < t_end) read_ids(kt + NW);
    // ---- K operand: key rows permuted so the S^T layout feeds P.V directly ------------
    // BIG: the tile's 64 rows are contiguous in one block; whole rows go to this wave's LDS
    // region first (read back below, once the V loads are in flight too).  Otherwise each
    // lane loads its rows' operand chunks itself.
    bf16x8 kf[2][2][D / 32];
    if (BIG) {
      const u16 *kb = P.k_pool + ((size_t)blk_t * P.Hkv + R.h) * head_stride +
                      (size_t)(k0 & bs_mask) * D;
#pragma unroll
      for (int j = 0; j < SK::NDMA; ++j) {
        const int row = SK::RPI * j + lane / SK::CPR;
        dma16_nt(kb + row * D + 8 * ((lane % SK::CPR) ^ swz_s<HD>(row)), kw_lds + 1024u * j);
      }
    } else {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const u16 *kp = P.k_pool + ((size_t)blk_k[kh][a] * P.Hkv + R.h) * head_stride +
                          (size_t)(k_key(k0, kh, a) & bs_mask) * D + 8 * g;
#pragma unroll
          for (int dc = 0; dc < D / 32; ++dc) kf[kh][a][dc] = as_bf16x8(ld16(kp + 32 * dc));
        }
    }
    // ---- V^T operand: 8 consecutive keys of one feature per lane ------------------------
    // In a block, V is stored as groups of 8 keys, each group feature-major with its 8 keys
    // adjacent (16 bytes).  One instruction (fixed kh, dt) reads, for each of the four lane
    // groups g, 16 consecutive features of one key group: four contiguous 256-byte runs.
    uint4 vr[2][D / 16];
    const u16 *vp[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      int keyc = k0 + 32 * kh + 8 * g, blk = blk_t;
      if (!BIG) {
        keyc = v_key(k0, kh);
        blk = blk_v[kh];
      }
      vp[kh] = P.v_pool + ((size_t)blk * P.Hkv + R.h) * head_stride +
               (size_t)(((keyc & bs_mask) >> 3) * D + r) * 8;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) vr[kh][dt] = ld16_nt(vp[kh] + 128 * dt);
    if (BIG) {
      // The DMAs were issued before the V loads: once every load of this wave is done, the
      // region holds the tile.  The empty asm keeps the V loads above the wait.
      asm volatile("" ::: "memory");
      wait_vm<0>();
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int key = 32 * kh + 8 * (r >> 2) + 4 * a + (r & 3);
#pragma unroll
          for (int dc = 0; dc < D / 32; ++dc)
            kf[kh][a][dc] = *reinterpret_cast<const bf16x8 *>(
                kw + key * D + 8 * ((4 * dc + g) ^ swz_s<HD>(key)));
        }
    }
    if (k0 + KT > R.khi) {  // keys at or past khi: zero V so stale bits cannot reach O
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int nvalid = min(max(R.khi - (k0 + 32 * kh + 8 * g), 0), 8);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) vr[kh][dt] = keep_first(vr[kh][dt], nvalid);
      }
    }
    // ---- S^T = K . Q^T, online softmax, O^T += V^T . P^T ------------------------------
    f32x4 st[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        st[kh][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) st[kh][a] = mfma_bf16(kf[kh][a][dc], qf[dc], st[kh][a]);
      }
    const bool need_mask = (k0 + KT > R.khi) || (k0 + KT - 1 > c + R.tok0);
    bf16x8 pf[2];
    online_softmax<HD>(st, need_mask, k0 + 8 * g, lim, R.khi, P.sl2, m_run, l_run, acc, pf);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = mfma_bf16(as_bf16x8(vr[kh][dt]), pf[kh], acc[dt]);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // ---- merge the waves through LDS ---------------------------------------------------
  // per-wave O^T dumps: wave w uses the w-th 8 KiB half-buffer of the ring (16 rows x 128
  // floats); the running maxima and sums go to the block-id array.  The dumps overlap other
  // waves' K regions, so every wave must be past its last tile first.
  __syncthreads();
  float *so_w = reinterpret_cast<float *>(S.base + w * STAGE_K);
  float *sm = reinterpret_cast<float *>(S.ids);                // [NW][16]
  float *sl = sm + NW * STREAM_ROWS;                           // [NW][16]
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4 *>(so_w + r * D + 16 * dt + 4 * g) = acc[dt];
  if (g == 0) {
    sm[w * STREAM_ROWS + r] = m_run;
    sl[w * STREAM_ROWS + r] = l_run;
  }
  __syncthreads();
  // one thread per (row, 8-feature chunk); threads past row 16 have nothing to merge
  const int row = threadIdx.x / (D / 8), chunk = threadIdx.x % (D / 8);
  if (row >= rows) return;
  float M = NEG_INF;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm[ww * STREAM_ROWS + row]);
  float Lsum = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float m = sm[ww * STREAM_ROWS + row];
    const float f = (m == NEG_INF) ? 0.f : fast_exp2(m - M);
    Lsum += sl[ww * STREAM_ROWS + row] * f;
    const float *src = reinterpret_cast<const float *>(S.base + ww * STAGE_K) + row * D + chunk * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] += src[i] * f;
  }
  if (R.group < 0) {
    const int t = qs + R.tok0 + row / P.G;
    if (t < P.num_tokens) store_out8<HD>(P, t, R.h * P.G + row % P.G, chunk * 8, o, 1.f / Lsum);
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

// ---------------------------------------------------------------------------------------
// MODE_TILE: up to TILE_ROWS query rows (chunk rows).  Wave w owns rows [32w, 32w+32) as one
// 32-row tile of the 32x32x16 MFMA.  Keys advance in 32-key stages; each stage's K [32 keys]
// [128] and V^T [128][32 keys] are fetched straight from HBM into LDS (global_load_lds_dwordx4,
// no register staging) through a ring of NSTAGE buffers, NSTAGE-1 stages ahead of the math, so
// the load latency hides behind three stages of MFMA work.  Every lane's source address is
// chosen so that the 1 KiB each wave instruction writes contiguously lands already swizzled.
//
// 32x32x16 layouts (k = 8*(l/32) + i for operand element i of lane l): A row m = l%32, B
// column n = l%32, result element j of lane l = C[8*(j/4) + 4*(l/32) + j%4][l%32].  Scores
// are S^T = K . Q^T; A row m reads key pi(m), pi swapping bits 2 and 3 of m, which leaves lane
// l with keys 8*(l/32) + (0..7) in elements 0..7 and 16 + 8*(l/32) + (0..7) in elements 8..15
// of its query row l%32: exactly the B operands (k = 16 keys each) of O^T += V^T . P^T.  So a
// row's softmax state lives in two lanes (l, l^32), and all 64 accumulators of a lane belong
// to one row, one scale factor.
// ---------------------------------------------------------------------------------------
static_assert(STREAM_ROWS * 128 * 4 <= stage_k(128) * 2 && STREAM_ROWS * 64 * 4 <= stage_k(64) * 2,
              "a wave's stream dump must fit a K array");
static_assert(NW * stage_k(128) <= NSTAGE * stage_elems(128) &&
                  NW * stage_k(64) <= NSTAGE * stage_elems(64),
              "every wave's stream dump must fit the ring");

// K stage: 16-byte chunk c of key row `key` sits at slot c ^ swz_k32<HD>(key).  The MFMA reads
// of 16 lanes (rows pi(m), m = 16i .. 16i+15, one chunk) then hit 16 distinct 16-byte slots of
// a 256-byte window: at HD 128 (256-byte rows) the swizzle takes 16 values; at HD 64 (128-byte
// rows, two per window) the row's parity picks the window half and the swizzle 8 values.
template <int HD>
__device__ __forceinline__ int swz_k32(int key) {
  if (HD == 128) return (key & 3) | ((key >> 1) & 4) | ((key << 1) & 8);
  return (key >> 1) & 7;
}
// V stage: the pool's own layout, [4 key groups][HD features][8 keys]: 16 lanes reading 16
// consecutive features of one key group read 256 contiguous bytes, so the operand reads are
// free of bank conflicts without a swizzle.
// pi: A row m of the score product reads physical key pi(m) of the stage (an involution)
__device__ __forceinline__ int key_perm32(int m) {
  return (m & ~12) | ((m >> 1) & 4) | ((m << 1) & 8);
}

// The stage ring: one workgroup-shared array, stage buffer i = K [32 keys][HD] followed by
// V [4 key groups][HD][8 keys].  Buffers are addressed as base + constant offset, so one set of per-lane
// address registers serves every buffer.
// The ring doubles as the stream records' per-wave K regions (128 KiB at HD 128).
constexpr int ring_elems(int hd) {
  return NSTAGE * stage_elems(hd) > NW * KEY_TILE * hd ? NSTAGE * stage_elems(hd) : NW * KEY_TILE * hd;
}
constexpr int MAX_IDS = 256;  // block ids of a tile record staged in LDS
static_assert(2 * NW * STREAM_ROWS <= MAX_IDS, "stream merge maxima and sums must fit");

template <int HD>
struct Lds {
  u16 *base;
  int *ids;  // MAX_IDS block ids
  __device__ u16 *k(int i) const { return base + i * stage_elems(HD); }
  __device__ u16 *v(int i) const { return base + i * stage_elems(HD) + stage_k(HD); }
};

// A stage is 2 * HD / 16 regions of 1 KiB: K regions first (HD / 16 of them, key rows of 2*HD
// bytes), then V regions (64 consecutive 16-byte (key group, feature) runs each: the stage's V
// is one contiguous piece of its block).  One wave instruction fills one region; wave w issues
// regions p * NW + w, p = 0 .. DPW - 1.
template <int HD>
struct Dma {
  static constexpr int K_REGIONS = HD / 16;
  static constexpr int DPW = 2 * K_REGIONS / NW;  // regions (instructions) per wave and stage
  static constexpr int ROWS_PER_K_REGION = 512 / HD;
  static_assert(DPW >= 1 && DPW * NW == 2 * K_REGIONS, "regions must split evenly over waves");
};

// Per-lane parts of a wave's LDS-DMA source addresses (bytes from the stage's first key in its
// block), constant over a record when a stage lies inside one block.
template <int HD>
struct DmaOffsets {
  uint32_t off[Dma<HD>::DPW];
  // the record's KV head in block 0 of each pool, and the bytes from one block to the next
  // (wave-uniform, so a stage's address is one scalar multiply-add away)
  const char *kh0, *vh0;
  uint64_t blk_bytes;
};

// region g of a stage, for this lane: a K region gives (key row, 16-byte chunk of its HD
// features); a V region gives (key group, feature) of the lane's 16-byte run
template <int HD>
__device__ __forceinline__ void dma_lane(int g, int lane, bool &isv, int &row, int &ch) {
  constexpr int KR = Dma<HD>::K_REGIONS, RPR = Dma<HD>::ROWS_PER_K_REGION;
  isv = g >= KR;
  if (!isv) {
    row = RPR * g + lane / (HD / 8);
    ch = (lane % (HD / 8)) ^ swz_k32<HD>(row);
  } else {
    const int unit = 64 * (g - KR) + lane;
    row = unit / HD;   // key group of the stage (0 .. 3)
    ch = unit % HD;    // feature
  }
}

template <int HD>
__device__ __forceinline__ DmaOffsets<HD> dma_offsets(int bs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  DmaOffsets<HD> o;
#pragma unroll
  for (int p = 0; p < Dma<HD>::DPW; ++p) {
    bool isv;
    int row, ch;
    dma_lane<HD>(p * NW + w, lane, isv, row, ch);
    o.off[p] = isv ? (uint32_t)(row * HD + ch) * 16u : (uint32_t)(row * HD + 8 * ch) * 2u;
  }
  return o;
}

// blk: the stage's block id, read ahead by the caller (used when a stage lies in one block)
template <int HD, int BSC>
__device__ __forceinline__ void issue_stage(const Params &P, const Rec &R, const int32_t *bt,
                                            int L, int k0, int blk, const DmaOffsets<HD> &o,
                                            u16 *buf) {
  constexpr int DPW = Dma<HD>::DPW, KR = Dma<HD>::K_REGIONS;
  const int lane = threadIdx.x & 63;
  // wave-uniform; the mask tells the compiler w < NW, so the K/V choice of a region folds
  // where it does not depend on the wave
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW - 1);
  const int bs_mask = P.bs - 1;
  const uint32_t lb = lds_addr_of(buf);
  if (BSC >= 1) {
    // a 32-key stage lies in one block: uniform base + per-lane offset
    const uint64_t hb = (uint64_t)(uint32_t)blk * o.blk_bytes;
    const uint32_t key_in_blk = (uint32_t)(k0 & bs_mask);
    const char *kb = o.kh0 + hb + key_in_blk * (uint32_t)(HD * 2);
    const char *vb = o.vh0 + hb + key_in_blk * (uint32_t)(HD * 2);  // 8-key groups of 16*HD bytes
#pragma unroll
    for (int p = 0; p < DPW; ++p) {
      const int g = p * NW + w;
      dma16(reinterpret_cast<const u16 *>((g >= KR ? vb : kb) + o.off[p]), lb + 1024u * g);
    }
    return;
  }
  const size_t head_stride = (size_t)P.bs * HD;
#pragma unroll
  for (int p = 0; p < DPW; ++p) {
    const int g = p * NW + w;
    bool isv;
    int row, ch;
    dma_lane<HD>(g, lane, isv, row, ch);
    if (!isv) {
      const int key = min(k0 + row, L - 1);
      const int blk = clamp_block(bt[key >> P.bs_log2], P.num_blocks);
      dma16(P.k_pool + ((size_t)blk * P.Hkv + R.h) * head_stride + (size_t)(key & bs_mask) * HD + 8 * ch,
            lb + 1024u * g);
    } else {
      const int key0 = min(k0 + 8 * row, (L - 1) & ~7);
      const int blk = clamp_block(bt[key0 >> P.bs_log2], P.num_blocks);
      dma16(P.v_pool + ((size_t)blk * P.Hkv + R.h) * head_stride +
                (size_t)(((key0 & bs_mask) >> 3) * HD + ch) * 8,
            lb + 1024u * g);
    }
  }
}

// Online softmax over one 32-key stage for this lane's query row: s[j] is the raw score of key
// key0 + 16*(j/8) + j%8 (key0 = k0 + 8*(l/32)).  Same arithmetic as online_softmax; P comes
// back as the two B operands of the P.V product.
__device__ __forceinline__ void mask_t32(f32x16 &s, int key0, int lim, int khi) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = key0 + 16 * (j / 8) + j % 8;
    if (key > lim || key >= khi) s[j] = NEG_INF;
  }
}

template <int HD>
__device__ __forceinline__ void online_softmax_t32(f32x16 &s, float sl2, float &m, float &l,
                                                   f32x16 *acc, bf16x8 (&pf)[2]) {
  float mx = s[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
  mx = pair_max(mx) * sl2;
  const bool upd = mx > m + LAZY_TAU;
  const float m_new = upd ? mx : m;
  const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
  const float alpha = fast_exp2(m - m_use);
  float p[16], psum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    p[j] = fast_exp2(fmaf(s[j], sl2, -m_use));
    psum += p[j];
  }
  l = l * alpha + psum;
  m = m_new;
  if (__ballot(upd)) {
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) acc[dt] *= alpha;
  }
  pf[0] = to_bf16x8(p);
  pf[1] = to_bf16x8(p + 8);
}

// The common case of a stage, in place: exponentials against the current running max m.  While
// every p stays within 2^LAZY_TAU -- which their sum bounds -- that max may stand, and the stage
// needs no max reduction and no rescale.  Returns false when it may not (a new max more than
// LAZY_TAU above m, the first stage with m = -inf giving an inf or NaN sum, an overflow); then
// s holds no scores any more and the caller redoes the stage with online_softmax_t32.
__device__ __forceinline__ bool softmax_t32_fast(f32x16 &s, float sl2, float m, float &l,
                                                 bf16x8 (&pf)[2]) {
  constexpr float P_CAP = 256.f;  // 2^LAZY_TAU
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    s[j] = fast_exp2(fmaf(s[j], sl2, -m));
    psum += s[j];
  }
  if (__ballot(!(psum <= P_CAP))) return false;
  l += psum;
  float p[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) p[j] = s[j];
  pf[0] = to_bf16x8(p);
  pf[1] = to_bf16x8(p + 8);
  return true;
}

template <int HD, int BSC>
__device__ void tile_record(const Params &P, const Rec &R, const Lds<HD> &S) {
  constexpr int D = HD;
  constexpr int DPW = Dma<HD>::DPW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, n = lane & 31;
  const int c = ldc(P.context_len, R.s), qs = ldc(P.query_start, R.s);
  const int L = c + ldc(P.n_query, R.s);
  const int rows = R.ntok * P.G;
  const int32_t *bt = P.block_table + (size_t)R.s * P.table_stride;

  // this wave's rows [32w, 32w + 32) (wave-uniform quantities, so their branches stay scalar)
  const bool active = rows > 32 * w;
  const int last_row = min(rows, 32 * w + 32) - 1;
  const int wave_lo = c + R.tok0 + (32 * w) / P.G;    // smallest key limit of the wave's rows
  const int wave_hi = c + R.tok0 + last_row / P.G;    // largest
  const int row = 32 * w + n;
  const int tok = R.tok0 + row / P.G;
  const int lim = c + tok;  // keys 0 .. lim are visible to this lane's row
  float m_run = NEG_INF, l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

  // LDS read offsets (elements) of this lane's MFMA operands within a stage
  const int krow = key_perm32(n), kswz = swz_k32<HD>(krow);

  const int s_begin = R.klo / KS, s_end = (R.khi + KS - 1) / KS, nst = s_end - s_begin;
  DmaOffsets<HD> doff = dma_offsets<HD>(P.bs);
  {
    const uint64_t head_bytes = (uint64_t)P.bs * D * 2;
    doff.kh0 = reinterpret_cast<const char *>(P.k_pool) + (uint64_t)R.h * head_bytes;
    doff.vh0 = reinterpret_cast<const char *>(P.v_pool) + (uint64_t)R.h * head_bytes;
    doff.blk_bytes = (uint64_t)P.Hkv * head_bytes;
  }

  // Keys at or past khi in the last stage may hold stale bits: zero their V so they cannot
  // reach O.  Called once that stage has landed for every wave.
  auto zero_tail = [&](u16 *Vl, int k0) {
    for (int idx = tid; idx < D * KS; idx += NT) {
      const int d = idx / KS, key = idx % KS;
      if (k0 + key >= R.khi) Vl[((key >> 3) * D + d) * 8 + (key & 7)] = 0;
    }
    __syncthreads();
  };
  bf16x8 qf[D / 16];  // B operands of the score product (loaded after the prologue below)
  // S^T = K . Q^T of one stage
  auto scores = [&](const u16 *Kl, f32x16 &out) {
    bf16x8 kf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      kf[st] = as_bf16x8(*reinterpret_cast<const uint4 *>(Kl + krow * D + 8 * ((2 * st + g) ^ kswz)));
#pragma unroll
    for (int j = 0; j < 16; ++j) out[j] = 0.f;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) out = mfma32_bf16(kf[st], qf[st], out);
  };

  f32x16 sc;  // scores of the current stage
  // block id of a stage (scalar load; stages of a block-size >= 32 cache lie in one block)
  // When the record's blocks fit, their ids are staged in LDS first: an LDS read of the next
  // id is cheap, while a scalar load's latency would surface at the next LDS wait (scalar and
  // LDS reads share one counter).
  const int b_first = R.klo >> P.bs_log2;
  const int n_ids = BSC >= 1 ? ((R.khi - 1) >> P.bs_log2) - b_first + 1 : 0;
  const bool ids_in_lds = n_ids <= MAX_IDS;
  if (BSC >= 1 && ids_in_lds) {
    for (int i = tid; i < n_ids; i += NT) S.ids[i] = clamp_block(bt[b_first + i], P.num_blocks);
    __syncthreads();
  }
  // (the LDS read lands in a vector register; it is made scalar only where it is used, one
  // stage later, so no wait for it stalls the loop)
  auto stage_block = [&](int i) {
    if (BSC == 0) return 0;
    const int b = ((s_begin + i) * KS) >> P.bs_log2;
    return ids_in_lds ? S.ids[b - b_first] : clamp_block(ldc(bt, b), P.num_blocks);
  };
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < nst)
      issue_stage<HD, BSC>(P, R, bt, L, (s_begin + i) * KS,
                           __builtin_amdgcn_readfirstlane(stage_block(i)), doff, S.k(i));
  // the block id of the next stage to fetch is read one stage ahead, so that the scalar
  // load's latency never stalls the loop
  int blk_next = NSTAGE - 1 < nst ? stage_block(NSTAGE - 1) : 0;
  // Q is loaded after the prologue stages; the compiler waits for it (and, loads completing
  // in order, for those stages) before its first use.
  {
    const int t = qs + tok, head = R.h * P.G + row % P.G;
    const bool ok = row < rows && t < P.num_tokens;
    // rows past the record read token 0 (always present) and are zeroed
    const u16 *qp = P.q + ((size_t)(ok ? t : 0) * P.Hq + (ok ? head : 0)) * D + 8 * g;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const uint4 v = ld16(qp + 16 * st);
      qf[st] = as_bf16x8(ok ? v : make_uint4(0, 0, 0, 0));
    }
  }

  // Steady state: the stages before the last NSTAGE and before any masked key (the record's
  // first row sees every key of them) need no mask, no tail zeroing, no refill or wait
  // bounds and no per-wave skip.  They run in a loop without those branches, NSTAGE at a
  // time; the general loop below takes the rest.
  int steady = 0;
  if (BSC >= 1 && ids_in_lds && rows > 32 * (NW - 1)) {
    const int unmasked = (c + R.tok0 + 1) / KS - s_begin;  // stages with k0 + KS - 1 <= first limit
    steady = max(0, min(unmasked, nst - NSTAGE));
    steady -= steady % NSTAGE;
  }
  for (int base = 0; base < steady; base += NSTAGE) {
#pragma unroll
    for (int u = 0; u < NSTAGE; ++u) {
      const int i = base + u;
      wait_dma(DPW * (NSTAGE - 2));
      stage_barrier();
      issue_stage<HD, BSC>(P, R, bt, L, (s_begin + i + NSTAGE - 1) * KS,
                           __builtin_amdgcn_readfirstlane(blk_next), doff,
                           S.k((u + NSTAGE - 1) % NSTAGE));
      blk_next = S.ids[(((s_begin + i + NSTAGE) * KS) >> P.bs_log2) - b_first];
      scores(S.k(u), sc);
      const u16 *Vl = S.v(u);
      bf16x8 vf[D / 32][2];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          vf[dt][h] = as_bf16x8(*reinterpret_cast<const uint4 *>(
              Vl + ((2 * h + g) * D + 32 * dt + n) * 8));
      bf16x8 pf[2];
      if (!softmax_t32_fast(sc, P.sl2, m_run, l_run, pf)) {
        scores(S.k(u), sc);
        online_softmax_t32<HD>(sc, P.sl2, m_run, l_run, acc, pf);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        acc[dt] = mfma32_bf16(vf[dt][0], pf[0], acc[dt]);
        acc[dt] = mfma32_bf16(vf[dt][1], pf[1], acc[dt]);
      }
    }
  }
  for (int base = steady; base < nst; base += NSTAGE) {
#pragma unroll
    for (int u = 0; u < NSTAGE; ++u) {   // unrolled so every stage buffer is a fixed array
      const int i = base + u;
      if (i >= nst) break;
      const int k0 = (s_begin + i) * KS;
      wait_dma(DPW * min(NSTAGE - 2, nst - 1 - i));  // this wave's loads of stage i landed
      stage_barrier();                              // ... and every other wave's
      if (i + NSTAGE - 1 < nst) {                   // refill the buffer stage i-1 used
        issue_stage<HD, BSC>(P, R, bt, L, (s_begin + i + NSTAGE - 1) * KS,
                             __builtin_amdgcn_readfirstlane(blk_next), doff,
                             S.k((u + NSTAGE - 1) % NSTAGE));
        if (i + NSTAGE < nst) blk_next = stage_block(i + NSTAGE);
      }
      if (k0 + KS > R.khi) zero_tail(S.v(u), k0);
      // a wave with no rows, or whose rows see none of these keys, has nothing to add
      if (active && k0 <= wave_hi) {
        scores(S.k(u), sc);
        const u16 *Vl = S.v(u);
        // V^T operands: feature 32*dt + n, keys 16*h + 8*g .. +7 (key group 2*h + g)
        bf16x8 vf[D / 32][2];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            vf[dt][h] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                Vl + ((2 * h + g) * D + 32 * dt + n) * 8));
        const bool need_mask = (k0 + KS > R.khi) || (k0 + KS - 1 > wave_lo);
        if (need_mask) mask_t32(sc, k0 + 8 * g, lim, R.khi);
        bf16x8 pf[2];
        if (!softmax_t32_fast(sc, P.sl2, m_run, l_run, pf)) {
          // rare: recompute the scores (the stage is still in LDS) and take the full path
          scores(S.k(u), sc);
          if (need_mask) mask_t32(sc, k0 + 8 * g, lim, R.khi);
          online_softmax_t32<HD>(sc, P.sl2, m_run, l_run, acc, pf);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          acc[dt] = mfma32_bf16(vf[dt][0], pf[0], acc[dt]);
          acc[dt] = mfma32_bf16(vf[dt][1], pf[1], acc[dt]);
        }
      }
    }
  }

  // ---- epilogue: normalise and store, or write the split partial ------------------------
  if (!active) return;
  l_run += __shfl_xor(l_run, 32, 64);
  if (row >= rows) return;
  // element j of acc[dt] is feature 32*dt + 8*(j/4) + 4*g + j%4 of this lane's row
  if (R.group < 0) {
    const int t = qs + tok;
    if (t >= P.num_tokens) return;
    const int head = R.h * P.G + row % P.G;
    const float inv = 1.f / l_run;
    u16 *op = P.out + ((size_t)t * P.Hq + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (__bf16)(acc[dt][4 * q4 + j] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * dt + 8 * q4) = v;
      }
  } else {
    float *sp = P.ws + R.poff + (int64_t)R.split * slot_floats(MODE_TILE, D);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4 *>(sp + row * D + 32 * dt + 8 * q4 + 4 * g) =
            f32x4{acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2], acc[dt][4 * q4 + 3]};
    if (g == 0) {
      sp[TILE_ROWS * D + row] = m_run;
      sp[TILE_ROWS * D + TILE_ROWS + row] = l_run;
    }
  }
}

// One launch serves every record of the pass: stream records (decode rows, HBM-bound) and
// tile records (chunk rows, MFMA-bound); the branch is uniform per workgroup.
// BSC: 0 = blocks of < 32 keys, 1 = blocks of 32 keys, 2 = blocks of >= 64 keys.
template <int HD, int BSC>
__global__ __launch_bounds__(NT, WG_PER_CU) void attention_bf16_kernel(Params P) {
  __shared__ __attribute__((aligned(16))) u16 ring[ring_elems(HD)];
  __shared__ int blk_ids[MAX_IDS];
  const Rec R = load_rec<HD>(P, blockIdx.x);
  if (R.s < 0 || !rec_fits_workspace<HD>(P, R)) return;  // never write outside the workspace
  Lds<HD> S;
  S.base = ring;
  S.ids = blk_ids;
  if (R.mode == MODE_STREAM)
    stream_record<HD, BSC == 2>(P, R, S);
  else
    tile_record<HD, BSC>(P, R, S);
}

// Merge records follow the attention records in the work list, one per split group.
template <int HD>
__global__ __launch_bounds__(NT) void attention_combine_kernel(Params P, int32_t first) {
  const Rec R = load_rec<HD>(P, first + blockIdx.x);
  if (R.s < 0 || R.group < 0 || !rec_fits_workspace<HD>(P, R)) return;
  merge_splits<HD>(P, R);
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
  const int vgl = min(bs_log2, 3);  // V slots in groups of min(8, bs)
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
      const int slot = kk & (bs - 1);
      const float *vp = v_pool + ((size_t)blk * Hkv + h) * HD * bs +
                        ((size_t)((slot >> vgl) * HD) << vgl) + (slot & ((1 << vgl) - 1));
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(pj, vp[(size_t)(lane + 64 * i) << vgl], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) out[((size_t)t * Hq + gq) * HD + lane + 64 * i] = acc[i] / l_run;
}

// ---------------------------------------------------------------------------------------
// KV append: one workgroup per (tile of TOK consecutive new tokens, KV head).  K rows are
// copied whole in 16-byte chunks (a K block row is contiguous).  V rows are staged in LDS and
// written as 8 tokens x 8 features per wave instruction: in the V layout (groups of 8 slots,
// each feature's 8 slots adjacent) the 8 consecutive tokens of a prompt chunk fill one group's
// 8 features as one 128-byte line, and a lone decode token's row touches 16 lines in all.
// TOK is 64, 32 or 16: the largest that still gives APPEND_MIN_WGS workgroups, so that a
// small pass (a few hundred decode tokens, or a 512-token chunk) still spreads over the chip.
// ---------------------------------------------------------------------------------------
constexpr int APPEND_THREADS = 256;
constexpr int64_t APPEND_MIN_WGS = 2048;  // eight per compute unit

template <typename T, int HD, int TOK>
__global__ __launch_bounds__(APPEND_THREADS) void kv_append_kernel(
    const int32_t *__restrict__ query_start, const int32_t *__restrict__ context_len,
    const int32_t *__restrict__ block_table, int32_t table_stride, int32_t num_seqs,
    int32_t num_tokens, const T *__restrict__ k_new, const T *__restrict__ v_new,
    T *__restrict__ k_pool, T *__restrict__ v_pool, int32_t Hkv, int32_t bs, int32_t bs_log2,
    int32_t num_blocks) {
  constexpr int VEC = 16 / sizeof(T);            // elements per 16-byte chunk
  constexpr int CPR = HD / VEC;                  // chunks per row
  constexpr int ROWP = HD + 4 / sizeof(T);       // LDS row padded by one dword
  __shared__ int dblk[TOK], dslot[TOK];
  __shared__ T vt[TOK * ROWP];
  const int t0 = blockIdx.x * TOK, h = blockIdx.y, tid = threadIdx.x;
  if (tid < TOK) {
    const int t = t0 + tid;
    int blk = -1, slot = 0;
    if (t < num_tokens) {
      int lo = 0, hi = num_seqs;  // s with query_start[s] <= t < query_start[s+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (query_start[mid] <= t) lo = mid; else hi = mid;
      }
      const int pos = context_len[lo] + (t - query_start[lo]);
      const int b = block_table[(size_t)lo * table_stride + (pos >> bs_log2)];
      if (b >= 0 && b < num_blocks) {  // validated on the host; never write out of range
        blk = b;
        slot = pos & (bs - 1);
      }
    }
    dblk[tid] = blk;
    dslot[tid] = slot;
  }
  __syncthreads();
  const size_t row_in = (size_t)Hkv * HD;  // elements per token in k_new / v_new
  for (int q = tid; q < TOK * CPR; q += APPEND_THREADS) {
    const int tok = q / CPR, c = q % CPR;
    const int blk = dblk[tok];
    if (blk < 0) continue;
    const uint4 v = *reinterpret_cast<const uint4 *>(k_new + (t0 + tok) * row_in + h * HD + c * VEC);
    *reinterpret_cast<uint4 *>(k_pool + (((size_t)blk * Hkv + h) * bs + dslot[tok]) * HD +
                               c * VEC) = v;
  }
  for (int q = tid; q < TOK * CPR; q += APPEND_THREADS) {
    const int tok = q / CPR, c = q % CPR;
    if (t0 + tok >= num_tokens) continue;
    const uint4 v = *reinterpret_cast<const uint4 *>(v_new + (t0 + tok) * row_in + h * HD + c * VEC);
    uint32_t *dst = reinterpret_cast<uint32_t *>(vt + tok * ROWP + c * VEC);
    dst[0] = v.x;
    dst[1] = v.y;
    dst[2] = v.z;
    dst[3] = v.w;
  }
  __syncthreads();
  const int vgl = min(bs_log2, 3);  // V slots in groups of min(8, bs)
  for (int idx = tid; idx < TOK * HD; idx += APPEND_THREADS) {
    const int u = idx >> 6, within = idx & 63;
    const int tok = 8 * (u % (TOK / 8)) + (within & 7);
    const int d = 8 * (u / (TOK / 8)) + (within >> 3);
    const int blk = dblk[tok];
    if (blk < 0) continue;
    const int slot = dslot[tok];
    v_pool[((size_t)blk * Hkv + h) * HD * bs + ((size_t)((slot >> vgl) * HD + d) << vgl) +
           (slot & ((1 << vgl) - 1))] = vt[tok * ROWP + d];
  }
}

}  // namespace

// =======================================================================================
// Launch of the attention records (one launch) and, when the plan splits, the merge records
// =======================================================================================
namespace {

template <int HD>
void launch_attention(const Params &P, int block_size, int32_t main_records, int32_t groups,
                      hipStream_t st) {
  if (block_size >= 64)
    hipLaunchKernelGGL((attention_bf16_kernel<HD, 2>), dim3(main_records), dim3(NT), 0, st, P);
  else if (block_size == 32)
    hipLaunchKernelGGL((attention_bf16_kernel<HD, 1>), dim3(main_records), dim3(NT), 0, st, P);
  else
    hipLaunchKernelGGL((attention_bf16_kernel<HD, 0>), dim3(main_records), dim3(NT), 0, st, P);
  if (groups > 0)
    hipLaunchKernelGGL((attention_combine_kernel<HD>), dim3(groups, TILE_ROWS / merge_rows(HD)),
                       dim3(NT), 0, st, P, main_records);
}

}  // namespace

// =======================================================================================
// Validation mode (FG_VALIDATE=1): copy the device descriptors (and work list) back on the
// caller's stream and check them on the host before launching anything.
// =======================================================================================
namespace {

bool validate_mode() {
  const char *v = getenv("FG_VALIDATE");
  return v && v[0] == '1' && v[1] == 0;
}

template <typename T>
fg_status copy_back(std::vector<T> &dst, const T *src, size_t n, hipStream_t st) {
  dst.resize(n ? n : 1);
  if (!n) return FG_OK;
  if (!src) return fail(FG_E_ARG, "descriptor array is null");
  const hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return fail(FG_E_HIP, "validation copy: %s", hipGetErrorString(e));
  return FG_OK;
}

// Host copy of a device batch (n_query derived from query_start when the device batch has
// none), checked with fg_validate_batch; the copies stay in `h` for further checks.
struct HostCopy {
  std::vector<int32_t> qs, nq, cl, bt;
  fg_ragged_batch b{};
};

fg_status validate_device_batch(const fg_cache *cache, const fg_ragged_batch *dev, hipStream_t st,
                                HostCopy &h) {
  const size_t S = (size_t)dev->num_seqs, W = (size_t)(dev->table_stride > 0 ? dev->table_stride : 0);
  fg_status r;
  if ((r = copy_back(h.qs, dev->query_start, S + 1, st)) != FG_OK) return r;
  if (dev->n_query && (r = copy_back(h.nq, dev->n_query, S, st)) != FG_OK) return r;
  if ((r = copy_back(h.cl, dev->context_len, S, st)) != FG_OK) return r;
  if ((r = copy_back(h.bt, dev->block_table, S * W, st)) != FG_OK) return r;
  const hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(FG_E_HIP, "validation sync: %s", hipGetErrorString(e));
  if (!dev->n_query) {
    h.nq.resize(S ? S : 1);
    for (size_t s = 0; s < S; ++s) h.nq[s] = h.qs[s + 1] - h.qs[s];
  }
  h.b = *dev;
  h.b.query_start = h.qs.data();
  h.b.n_query = h.nq.data();
  h.b.context_len = h.cl.data();
  h.b.block_table = h.bt.data();
  h.b.seq_index = nullptr;
  h.b.seq_id = nullptr;
  return fg_validate_batch(cache, &h.b);
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
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(FG_E_ARG, "k_new and v_new must be 16-byte aligned");
  const fg_cache_config &c = cache->cfg;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    HostCopy h;
    const fg_status r = validate_device_batch(cache, dev, st, h);
    if (r != FG_OK) return r;
  }
  int tok = 64;  // largest tile that still fills the chip (see kv_append_kernel)
  while (tok > 16 && (int64_t)((dev->num_tokens + tok - 1) / tok) * c.num_kv_heads < APPEND_MIN_WGS)
    tok /= 2;
  const dim3 grid((dev->num_tokens + tok - 1) / tok, c.num_kv_heads);
  const dim3 block(APPEND_THREADS);
#define FG_APPEND_TOK(T, HD, TOKC)                                                             \
  hipLaunchKernelGGL((kv_append_kernel<T, HD, TOKC>), grid, block, 0, st, dev->query_start,     \
                     dev->context_len, dev->block_table, dev->table_stride, dev->num_seqs,     \
                     dev->num_tokens, (const T *)k_new, (const T *)v_new, (T *)cache->k_pool,  \
                     (T *)cache->v_pool, c.num_kv_heads, c.block_size, cache->bs_log2,         \
                     c.num_blocks)
#define FG_APPEND(T, HD)                                                                      \
  do {                                                                                        \
    if (tok == 64) FG_APPEND_TOK(T, HD, 64);                                                  \
    else if (tok == 32) FG_APPEND_TOK(T, HD, 32);                                             \
    else FG_APPEND_TOK(T, HD, 16);                                                            \
  } while (0)
  if (c.dtype == FG_BF16 && c.head_dim == 64)
    FG_APPEND(u16, 64);
  else if (c.dtype == FG_BF16)
    FG_APPEND(u16, 128);
  else if (c.head_dim == 64)
    FG_APPEND(float, 64);
  else
    FG_APPEND(float, 128);
#undef FG_APPEND
#undef FG_APPEND_TOK
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_E_HIP, "kv_append launch: %s", hipGetErrorString(e));
  return FG_OK;
}

}  // extern "C"

namespace {

// The attention call with a given workspace; `validate`: honour FG_VALIDATE.
fg_status attention_impl(const fg_cache *cache, const fg_ragged_batch *dev,
                         const fg_attention_plan_info *plan, const int32_t *work_dev,
                         const void *q, int32_t num_q_heads, float scale, void *out,
                         void *workspace, size_t workspace_bytes, void *stream, bool validate) {
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
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(workspace)) & 15)
    return fail(FG_E_ARG, "q, out and workspace must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (validate && validate_mode()) {
    HostCopy h;
    fg_status r = validate_device_batch(cache, dev, st, h);
    if (r != FG_OK) return r;
    if (c.dtype == FG_BF16) {
      if (!plan) return fail(FG_E_ARG, "bf16 attention needs the plan info");
      std::vector<int32_t> work;
      if ((r = copy_back(work, work_dev, (size_t)(plan->work_ints > 0 ? plan->work_ints : 0), st)) != FG_OK)
        return r;
      const hipError_t e = hipStreamSynchronize(st);
      if (e != hipSuccess) return fail(FG_E_HIP, "validation sync: %s", hipGetErrorString(e));
      h.b.num_tokens = dev->num_tokens;
      if ((r = fg_validate_work(cache, &h.b, plan, work.data(), workspace_bytes)) != FG_OK) return r;
    }
  }
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
    if (plan->num_work < 1 || !work_dev || plan->num_groups < 0 ||
        plan->num_groups >= plan->num_work || plan->num_items < 1 ||
        plan->work_ints != plan->num_items * FG_ITEM_INTS + plan->num_work)
      return fail(FG_E_ARG, "empty, null or inconsistent work list");
    if (plan->workspace_bytes > 0 && (!workspace || workspace_bytes < (size_t)plan->workspace_bytes))
      return fail(FG_E_WORKSPACE, "workspace of %zu bytes, plan needs %lld", workspace_bytes,
                  (long long)plan->workspace_bytes);
    if (c.head_dim != 64 && c.head_dim != 128)
      return fail(FG_E_UNSUPPORTED, "bf16 head_dim %d", c.head_dim);
    if (c.block_size < 8)
      return fail(FG_E_UNSUPPORTED, "bf16 attention reads 8-key runs: block_size %d < 8",
                  c.block_size);
    Params P;
    P.items = work_dev;
    P.codes = work_dev + (size_t)plan->num_items * FG_ITEM_INTS;
    P.num_items = plan->num_items;
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
    P.ws_floats = (int64_t)(workspace ? workspace_bytes / 4 : 0);
    P.Hq = num_q_heads;
    P.Hkv = c.num_kv_heads;
    P.G = num_q_heads / c.num_kv_heads;
    P.bs = c.block_size;
    P.bs_log2 = cache->bs_log2;
    P.num_blocks = c.num_blocks;
    P.sl2 = scale * LOG2E;
    const int32_t main_records = plan->num_work - plan->num_groups;
    if (c.head_dim == 128)
      launch_attention<128>(P, c.block_size, main_records, plan->num_groups, st);
    else
      launch_attention<64>(P, c.block_size, main_records, plan->num_groups, st);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_E_HIP, "attention launch: %s", hipGetErrorString(e));
  return FG_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Fixed scratch for fg_ragged_attention_noalloc: the split partials live in this file-scope
// device array instead of a caller workspace.  Each device holds its own copy (for the life
// of the process).  Host code never passes the array's name to a kernel (on the host it is
// only a stand-in symbol); it uses the device address hipGetSymbolAddress returns, looked up
// once per device on the entry point's first call there.
// ---------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[FG_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

fg_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FG_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(FG_E_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FG_E_HIP, "hipGetSymbolAddress of the fixed scratch: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FG_OK;
}

}  // namespace

extern "C" {

fg_status fg_ragged_attention(const fg_cache *cache, const fg_ragged_batch *dev,
                              const fg_attention_plan_info *plan, const int32_t *work_dev,
                              const void *q, int32_t num_q_heads, float scale, void *out,
                              void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  return attention_impl(cache, dev, plan, work_dev, q, num_q_heads, scale, out, workspace,
                        workspace_bytes, stream, true);
}

fg_status fg_ragged_attention_noalloc(const fg_cache *cache, const fg_ragged_batch *dev,
                                      const fg_attention_plan_info *plan,
                                      const int32_t *work_dev, const void *q,
                                      int32_t num_q_heads, float scale, void *out,
                                      void *stream) {
  clear_error();
  if (plan && plan->workspace_bytes > (int64_t)FG_NOALLOC_WORKSPACE_BYTES)
    return fail(FG_E_WORKSPACE,
                "plan needs %lld bytes of split partials, more than the %lld-byte fixed scratch "
                "of fg_ragged_attention_noalloc (use fg_ragged_attention with a workspace, or "
                "plan for fewer compute units)",
                (long long)plan->workspace_bytes, (long long)FG_NOALLOC_WORKSPACE_BYTES);
  void *ws = nullptr;
  if (plan && plan->workspace_bytes > 0) {
    const fg_status r = scratch_address(&ws);
    if (r != FG_OK) return r;
  }
  return attention_impl(cache, dev, plan, work_dev, q, num_q_heads, scale, out, ws,
                        ws ? (size_t)FG_NOALLOC_WORKSPACE_BYTES : 0, stream, false);
}

}  // extern "C"
