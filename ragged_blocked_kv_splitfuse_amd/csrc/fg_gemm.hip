// Dense projections either side of attention, as a gfx950 bf16 MFMA GEMM of this library.
//
// The QKV projection produces the rows fg_kv_append stores and fg_ragged_attention reads; the
// output projection maps attention's rows back (DeepSpeed-FastGen paper card by Holmes et al.
// 2024, "Key points": the kernels around attention come from FasterTransformer).  Both are
//     y[T][N] = x[T][K] . w[N][K]^T        (w in the [out][in] layout of a linear layer)
// with bf16 inputs, fp32 accumulation and one round-to-nearest-even to bf16 per output.
//
// Design (CDNA4): a workgroup of WF x WT waves computes a (32*TT*WT tokens) x (32*FT*WF
// features) tile; each wave owns FT x TT tiles of the 32x32x16 bf16 MFMA.  Four-wave tiles run
// two workgroups per CU; the 256 x 256 tile is eight waves (4 x 2, 2 x 4 MFMA tiles each), so
// that every SIMD has two waves to issue its matrix instructions from.  The MFMA computes the
// transposed product C^T = W . X^T (A operand: 32 weight rows, B operand: 32 token rows; both
// rows are contiguous along K, so every operand is one 16-byte load), which leaves each lane
// with runs of four consecutive output features of one token: 8-byte stores into the output
// matrix those columns belong to (y, or q, k and v for the fused QKV projection).  The
// inner dimension advances in BK-element stages; each stage's weight and token rows go from
// memory straight into LDS with 16-byte LDS-DMA loads through an NSTG-deep ring, each buffer
// refilled as soon as every wave has read it, swizzled so that the operand reads are free of
// bank conflicts.  The operand reads run one MFMA k-step ahead of the products (two register
// sets), interleaved with them, so the matrix cores do not wait for LDS.  The host
// picks the tile by the rounds of workgroups each would need (ragged token counts run from a
// few rows to thousands).  Tiles are placed per XCD where the shape allows (workgroup
// b runs on XCD b % 8): each XCD takes a contiguous eighth of the output features, so its L2
// holds that eighth of the weights while the token rows stream.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fg_internal.h"

using fgi::fail;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int NUM_XCD = 8;

// WF x WT waves over the workgroup's tile (wave-major along tokens), each owning FT x TT tiles
// of the 32x32x16 MFMA.
template <int FT, int TT, int BK, int WF, int WT>
struct Tile {
  static constexpr int NWV = WF * WT;                // waves per workgroup
  static constexpr int THREADS = 64 * NWV;
  static constexpr int BN = 32 * FT * WF;            // output features per workgroup
  static constexpr int BM = 32 * TT * WT;            // tokens per workgroup
  static constexpr int ROW = BK * 2;                 // bytes per tile row of a stage
  static constexpr int CH = BK / 8;                  // 16-byte chunks per row
  static constexpr int STAGE = (BN + BM) * ROW;      // weight rows, then token rows
  static constexpr int REGIONS = STAGE / 1024;       // 1 KiB per LDS-DMA wave instruction
  static constexpr int W_REGIONS = BN * ROW / 1024;  // regions of weight rows
  static constexpr int RPR = 1024 / ROW;             // rows per region
  static constexpr int DPW = REGIONS / NWV;          // LDS-DMA instructions per wave and stage
  // Workgroups per compute unit: eight waves (two per SIMD) fill a CU alone; four-wave tiles
  // run two workgroups per CU.
  static constexpr int WGS = NWV == 8 ? 1 : 2;
  // ring depth: three stages where the workgroups of a compute unit still fit in LDS, else two
  static constexpr int LDS_PER_WG = (WGS == 1 ? 144 : 80) * 1024;
  static constexpr int NSTG = 3 * STAGE <= LDS_PER_WG ? 3 : 2;
  static_assert(DPW * NWV == REGIONS && W_REGIONS * 1024 == BN * ROW, "regions");
  static_assert(3 * DPW <= 63, "the stage waits count LDS-DMA loads in vmcnt's range");
  static_assert(NSTG * STAGE <= LDS_PER_WG, "the ring must fit the workgroups of a CU");
};

// 16-byte chunk c of tile row r sits at slot c ^ swz(r): the 16 lanes of one operand read (16
// consecutive rows, one chunk) then hit 16 distinct 16-byte slots of a 256-byte window.  Rows
// of 128 bytes (BK 64): two rows per window, the swizzle takes 8 values.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  static_assert(BK == 64, "stages are 64 inner elements wide");
  return (r >> 1) & 7;
}

// Where the product's output columns go: columns [col0[s], col0[s + 1]) form row-major matrix
// s, y[s][T][col0[s + 1] - col0[s]] (one matrix for a plain linear layer; Q, K and V for the
// fused QKV projection).  Every boundary is a multiple of the tile widths in use, so the
// columns a workgroup writes lie in one matrix.
struct OutSeg {
  u16 *y[3];
  int col0[4];  // col0[0] = 0; unused boundaries equal N
};

// element (t, f) of the output, f a column of the whole product
__device__ __forceinline__ u16 *out_at(const OutSeg &o, int t, int f) {
  const int s = (f >= o.col0[1]) + (f >= o.col0[2]);
  return o.y[s] + (size_t)t * (o.col0[s + 1] - o.col0[s]) + (f - o.col0[s]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One wave instruction: 16 bytes per lane from global memory to LDS at lds + 16*lane (the LDS
// base goes in M0, through the operand).  Untracked by the compiler; the kernel waits for these
// with explicit vmcnt counts and orders them against LDS reads with barriers.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt encoding (gfx9): vmcnt = bits 3:0 (+ bits 15:14), expcnt 6:4, lgkmcnt 11:8
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int FT, int TT, int BK, int WF, int WT>
__global__ __launch_bounds__(64 * WF * WT, WF * WT == 8 ? 1 : 2) void gemm_nt_bf16_kernel(const u16 *__restrict__ x,
                                                             const u16 *__restrict__ w,
                                                             const OutSeg o, int T, int K,
                                                             int N, int xcd_split) {
  using Tl = Tile<FT, TT, BK, WF, WT>;
  constexpr int BN = Tl::BN, BM = Tl::BM, ROW = Tl::ROW, DPW = Tl::DPW, NSTG = Tl::NSTG;
  constexpr int NWV = Tl::NWV;
  __shared__ __attribute__((aligned(16))) unsigned char ring[NSTG * Tl::STAGE];
  const int NT = N / BN;
  int mt, nt;
  if (xcd_split) {  // XCD x takes column tiles [x * NT/8, (x+1) * NT/8), all row tiles
    const int per = NT / NUM_XCD, b = blockIdx.x;
    const int x8 = b % NUM_XCD, idx = b / NUM_XCD;
    mt = idx / per;
    nt = x8 * per + idx % per;
  } else {
    mt = blockIdx.x / NT;
    nt = blockIdx.x % NT;
  }
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wv / WT, wt = wv % WT;  // this wave's features (wf) and tokens (wt)
  const int f_base = nt * BN, t_base = mt * BM;

  // LDS-DMA sources of this lane: wave wv fills regions p*NWV + wv; a region is RPR tile rows
  // (weight rows first, then token rows), lane -> (row, 16-byte slot)
  const u16 *src[DPW];
#pragma unroll
  for (int p = 0; p < DPW; ++p) {
    const int reg = p * NWV + wv;
    const bool wrow = reg < Tl::W_REGIONS;
    const int rr = Tl::RPR * (wrow ? reg : reg - Tl::W_REGIONS) + lane / Tl::CH;
    const int c = (lane % Tl::CH) ^ swz<BK>(rr);
    if (wrow)
      src[p] = w + (size_t)(f_base + rr) * K + 8 * c;
    else
      src[p] = x + (size_t)min(t_base + rr, T - 1) * K + 8 * c;  // rows past T: read, unused
  }
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)ring;
  auto issue = [&](int s) {  // stage s into buffer s % NSTG
    const uint32_t base = lds0 + (uint32_t)(s % NSTG) * Tl::STAGE;
#pragma unroll
    for (int p = 0; p < DPW; ++p) dma16(src[p] + (size_t)s * BK, base + 1024u * (p * NWV + wv));
  };

  // operand rows of this lane: weights 32*FT*wf + 32*i + n, tokens 32*TT*wt + 32*j + n
  int arow[FT], brow[TT];
#pragma unroll
  for (int i = 0; i < FT; ++i) arow[i] = 32 * FT * wf + 32 * i + n;
#pragma unroll
  for (int j = 0; j < TT; ++j) brow[j] = 32 * TT * wt + 32 * j + n;
  f32x16 acc[FT][TT];
#pragma unroll
  for (int i = 0; i < FT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nst = K / BK;
  constexpr int KS = BK / 16;  // MFMA k-steps per stage (even)
  static_assert(KS % 2 == 0, "operand double buffer alternates within a stage");
  // wait until at most n stages of this wave's LDS-DMA loads are in flight (n in 0 .. 3)
  auto wait_stages = [&](int n) {
    if (n >= 3) wait_vm<3 * DPW>();
    else if (n == 2) wait_vm<2 * DPW>();
    else if (n == 1) wait_vm<DPW>();
    else wait_vm<0>();
  };
  // operands of k-step ks of stage s into register set r
  bf16x8 a[2][FT], b[2][TT];
  auto read_ops = [&](int s, int ks, int r) {
    const unsigned char *wb = ring + (s % NSTG) * Tl::STAGE;
    const unsigned char *xb = wb + BN * ROW;
    const int c = 2 * ks + g;  // this lane's 8 inner elements: chunk c of its row
#pragma unroll
    for (int i = 0; i < FT; ++i)
      a[r][i] = *reinterpret_cast<const bf16x8 *>(wb + arow[i] * ROW + 16 * (c ^ swz<BK>(arow[i])));
#pragma unroll
    for (int j = 0; j < TT; ++j)
      b[r][j] = *reinterpret_cast<const bf16x8 *>(xb + brow[j] * ROW + 16 * (c ^ swz<BK>(brow[j])));
  };
  // the products of one k-step, with the next k-step's operand reads (issued just before)
  // placed between its first products, one after each, so that they land well before the
  // next k-step needs them
  auto products = [&](int r) {
#pragma unroll
    for (int i = 0; i < FT; ++i)
#pragma unroll
      for (int j = 0; j < TT; ++j) acc[i][j] = mfma32(a[r][i], b[r][j], acc[i][j]);
#pragma unroll
    for (int q = 0; q < FT + TT; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  };

  // Every buffer of the ring is filled ahead; stage s's buffer is refilled (stage s + NSTG)
  // once every wave has read all of stage s, i.e. after the barrier that also makes stage
  // s + 1 visible.  The operand reads run one k-step ahead of the products, across that
  // barrier too, so the matrix cores do not wait for LDS between k-steps.
#pragma unroll
  for (int s = 0; s < NSTG; ++s)
    if (s < nst) issue(s);
  wait_stages(min(nst - 1, NSTG - 1));
  barrier();
  read_ops(0, 0, 0);
  for (int s = 0; s < nst; ++s) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
        read_ops(s, ks + 1, cur ^ 1);
      } else {
        // stage s fully read by this wave (its last operands are in registers), stage s + 1
        // landed for this wave; the barrier extends both to every wave.  After the last stage
        // this reads a stale buffer into registers that are never used, so that no branch
        // leaves the compiler unsure which LDS reads are still in flight.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        wait_stages(max(0, min(nst - 2 - s, NSTG - 2)));
        barrier();
        if (s + NSTG < nst) issue(s + NSTG);
        read_ops(s + 1, 0, cur ^ 1);
      }
      products(cur);
    }
  }

  // epilogue: element e of acc[i][j] is feature 8*(e/4) + 4*g + e%4 of the i-th 32-feature
  // block, for token n of the j-th 32-token block
#pragma unroll
  for (int j = 0; j < TT; ++j) {
    const int t = t_base + 32 * TT * wt + 32 * j + n;
    if (t >= T) continue;
    u16 *yr = out_at(o, t, f_base + 32 * FT * wf + 4 * g);
#pragma unroll
    for (int i = 0; i < FT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[i][j][4 * q + e];
        *reinterpret_cast<bf16x4 *>(yr + 32 * i + 8 * q) = v;
      }
  }
}

template <int FT, int TT, int BK, int WF, int WT>
void launch(const u16 *x, const u16 *w, const OutSeg &y, int T, int K, int N, hipStream_t st) {
  using Tl = Tile<FT, TT, BK, WF, WT>;
  const int NT = N / Tl::BN, MT = (T + Tl::BM - 1) / Tl::BM;
  hipLaunchKernelGGL((gemm_nt_bf16_kernel<FT, TT, BK, WF, WT>), dim3((unsigned)(NT * MT)),
                     dim3(Tl::THREADS), 0,
                     st, x, w, y, T, K, N, NT % NUM_XCD == 0 ? 1 : 0);
}

// ---------------------------------------------------------------------------------------
// Few token rows (T <= 64, the passes of a serving loop that carry only decode tokens): the
// product is a stream of the weights, read once, against a handful of token rows that every
// workgroup reads from L2.  One workgroup of eight waves per 16 output features (N / 16
// workgroups: 256 for N = 4096).  The inner dimension advances in SKK-element stages; a stage
// holds the 16 weight rows and the 16 * NT token rows (rows past T repeat row T-1, unused) and
// goes to LDS by LDS-DMA in whole rows, three stages deep: loaded straight into MFMA operand
// registers, each instruction would read half of 16 cache lines, at about a third of the rate
// of whole lines.  Wave w takes the k-steps w, w + 8, ... of every stage (16x16x32 bf16 MFMA,
// C^T = W . X^T); the eight partial tiles are summed through LDS in wave order (deterministic),
// rounded once to bf16 and stored.
// ---------------------------------------------------------------------------------------
constexpr int SK_THREADS = 512;  // eight waves
constexpr int SK_WAVES = SK_THREADS / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int NT>
struct Skinny {
  static constexpr int SKK = NT <= 2 ? 512 : 256;  // inner elements per stage
  static constexpr int ROWS = 16 + 16 * NT;         // weight rows, then token rows
  static constexpr int ROWB = SKK * 2;              // bytes per stage row
  static constexpr int STAGE = ROWS * ROWB;
  static constexpr int NI = STAGE / 1024;           // LDS-DMA instructions per stage
  static constexpr int DPW = NI / SK_WAVES;         // ... per wave
  static constexpr int RPI = 1024 / ROWB;           // rows per instruction
  static constexpr int KSW = SKK / 32 / SK_WAVES;   // k-steps per wave and stage
  static constexpr int NSTG = 3;
  static_assert(DPW * SK_WAVES == NI && KSW >= 1, "stage split");
  static_assert(NSTG * STAGE <= 144 * 1024, "ring");
};

// 16-byte chunk c of stage row r sits at slot c ^ (r & 15): 16 lanes reading one chunk of 16
// consecutive rows hit 16 distinct slots of a 256-byte window.
template <int NT>
__global__ __launch_bounds__(SK_THREADS) void gemm_skinny_bf16_kernel(const u16 *__restrict__ x,
                                                                       const u16 *__restrict__ w,
                                                                       const OutSeg o, int T,
                                                                       int K, int N) {
  using Sk = Skinny<NT>;
  constexpr int ROWB = Sk::ROWB, DPW = Sk::DPW, NSTG = Sk::NSTG;
  __shared__ __attribute__((aligned(16))) unsigned char ring[NSTG * Sk::STAGE];
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int f0 = blockIdx.x * 16;
  // LDS-DMA sources of this lane: instruction p*8 + wv fills stage rows RPI*(p*8+wv) ..
  const u16 *src[DPW];
#pragma unroll
  for (int p = 0; p < DPW; ++p) {
    const int ins = p * SK_WAVES + wv;
    const int row = Sk::RPI * ins + lane / (ROWB / 16);
    const int c = (lane % (ROWB / 16)) ^ (row & 15);
    src[p] = row < 16 ? w + (size_t)(f0 + row) * K + 8 * c
                      : x + (size_t)min(row - 16, T - 1) * K + 8 * c;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)ring;
  auto issue = [&](int s) {
    const uint32_t base = lds0 + (uint32_t)(s % NSTG) * Sk::STAGE;
#pragma unroll
    for (int p = 0; p < DPW; ++p)
      dma16(src[p] + (size_t)s * Sk::SKK, base + 1024u * (p * SK_WAVES + wv));
  };
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = K / Sk::SKK;
#pragma unroll
  for (int s = 0; s < NSTG - 1; ++s)
    if (s < nst) issue(s);
  for (int s = 0; s < nst; ++s) {
    // this wave's loads of stage s landed (the next stage may still be in flight) ...
    if (s + 1 < nst) wait_vm<DPW>();
    else wait_vm<0>();
    barrier();  // ... and every wave's; stage s-1 is consumed, its buffer free
    if (s + NSTG - 1 < nst) issue(s + NSTG - 1);
    const unsigned char *sb = ring + (s % NSTG) * Sk::STAGE;
#pragma unroll
    for (int q = 0; q < Sk::KSW; ++q) {
      const int c = 4 * (q * SK_WAVES + wv) + g;  // chunk of this lane's 8 inner elements
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sb + r * ROWB + 16 * (c ^ r));
      bf16x8 b[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = 16 + 16 * j + r;
        b[j] = *reinterpret_cast<const bf16x8 *>(sb + row * ROWB + 16 * (c ^ (row & 15)));
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mfma16(a, b[j], acc[j]);
    }
  }
  barrier();  // every wave is done with the ring
  // element e of acc[j] (lane l): feature 4*(l/16) + e, token 16*j + l%16
  float *part = reinterpret_cast<float *>(ring);  // [wave][NT][64 lanes][4]
#pragma unroll
  for (int j = 0; j < NT; ++j)
    *reinterpret_cast<f32x4 *>(part + ((wv * NT + j) * 64 + lane) * 4) = acc[j];
  __syncthreads();
  for (int q = threadIdx.x; q < NT * 64; q += SK_THREADS) {  // (tile, lane) pairs
    const int j = q >> 6, l = q & 63;
    const int t = 16 * j + (l & 15);
    f32x4 sum = *reinterpret_cast<const f32x4 *>(part + (j * 64 + l) * 4);
#pragma unroll
    for (int u = 1; u < SK_WAVES; ++u)
      sum += *reinterpret_cast<const f32x4 *>(part + ((u * NT + j) * 64 + l) * 4);
    if (t < T) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)sum[e];
      *reinterpret_cast<bf16x4 *>(out_at(o, t, f0 + 4 * (l >> 4))) = v;
    }
  }
}

template <int NT>
void launch_skinny(const u16 *x, const u16 *w, const OutSeg &y, int T, int K, int N,
                   hipStream_t st) {
  hipLaunchKernelGGL((gemm_skinny_bf16_kernel<NT>), dim3((unsigned)(N / 16)), dim3(SK_THREADS),
                     0, st, x, w, y, T, K, N);
}

// Picks the kernel and tile for T x N x K and launches it.  wide_ok: every output matrix's
// width is a multiple of 256 (the 256 x 256 tile may be used).
fg_status run_linear(const u16 *xp, const u16 *wp, const OutSeg &o, int T, int K, int N,
                     bool wide_ok, hipStream_t st) {
  // Between the eight-wave 256 x 256 tile (one workgroup per compute unit, the chip has 256)
  // and the four-wave 128 x 128 tile (two per CU), by rounds of workgroups: a full round takes
  // ~111 us of the former and ~64 us of the latter at K = 4096 (both scale with K), so the
  // 256 x 256 tile is taken when its rounds cost no more (partly empty rounds and half-empty
  // token tiles count as full ones).  Measured on ~40 projection shapes (K 4096; N 1024 to
  // 12288; T 512 to 4100) this picks the faster of the two everywhere but at ties (within 4%);
  // e.g. T = 1040, N = 12288: 114 against 124 us (one round against two), T = 640: 67 us on
  // 128 x 128 against 93 (one round each).  Below that, 128 x 64 tiles when 128 x 128 would
  // not put a workgroup on every CU.  (The four-wave 256 x 256 form, one wave per SIMD, was
  // 7-16% slower than the eight-wave one; 256 x 128 tiles are now slower than 128 x 128.)
  // Up to 64 token rows: the weight-streaming kernel (whole stages of 512 or 256 inner
  // elements).
  if (T <= 64 && K % 512 == 0) {
    if (T <= 16) launch_skinny<1>(xp, wp, o, T, K, N, st);
    else if (T <= 32) launch_skinny<2>(xp, wp, o, T, K, N, st);
    else if (T <= 48) launch_skinny<3>(xp, wp, o, T, K, N, st);
    else launch_skinny<4>(xp, wp, o, T, K, N, st);
  } else {
    const auto tiles = [&](int bm, int bn) { return (int64_t)((T + bm - 1) / bm) * (N / bn); };
    constexpr int64_t CUS = 256, ROUND_256_US = 111, ROUND_128_US = 64;
    const int64_t t256 = wide_ok ? tiles(256, 256) : 0, t128 = tiles(128, 128);
    const int64_t rounds_256 = (t256 + CUS - 1) / CUS, rounds_128 = (t128 + 2 * CUS - 1) / (2 * CUS);
    if (t256 > 0 && ROUND_256_US * rounds_256 <= ROUND_128_US * rounds_128)
      launch<2, 4, 64, 4, 2>(xp, wp, o, T, K, N, st);
    else if (t128 > CUS)
      launch<2, 2, 64, 2, 2>(xp, wp, o, T, K, N, st);
    else
      launch<2, 1, 64, 2, 2>(xp, wp, o, T, K, N, st);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_E_HIP, "GEMM launch: %s", hipGetErrorString(e));
  return FG_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" fg_status fg_linear_bf16(const void *x, const void *w, void *y, int32_t T, int32_t K,
                                    int32_t N, void *stream) {
  fgi::clear_error();
  if (T < 0 || K < 1 || N < 1) return fail(FG_E_ARG, "sizes T=%d K=%d N=%d", T, K, N);
  if (T == 0) return FG_OK;
  if (!x || !w || !y) return fail(FG_E_ARG, "null x, w or y");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y))
    return fail(FG_E_ARG, "x, w and y must be 16-byte aligned");
  if (N % 128 || K % 64)
    return fail(FG_E_UNSUPPORTED, "the GEMM tiles need N %% 128 == 0 and K %% 64 == 0 (N=%d, K=%d)",
                N, K);
  if ((int64_t)T * (N / 128) > INT32_MAX) return fail(FG_E_UNSUPPORTED, "too many tiles");
  OutSeg o;
  o.y[0] = o.y[1] = o.y[2] = (u16 *)y;
  o.col0[0] = 0;
  o.col0[1] = o.col0[2] = o.col0[3] = N;
  return run_linear((const u16 *)x, (const u16 *)w, o, T, K, N, N % 256 == 0,
                    reinterpret_cast<hipStream_t>(stream));
}

extern "C" fg_status fg_linear_qkv_bf16(const void *x, const void *w_qkv, void *q, void *k,
                                        void *v, int32_t T, int32_t K, int32_t Nq, int32_t Nkv,
                                        void *stream) {
  fgi::clear_error();
  if (T < 0 || K < 1 || Nq < 1 || Nkv < 1)
    return fail(FG_E_ARG, "sizes T=%d K=%d Nq=%d Nkv=%d", T, K, Nq, Nkv);
  if (T == 0) return FG_OK;
  if (!x || !w_qkv || !q || !k || !v) return fail(FG_E_ARG, "null x, w_qkv, q, k or v");
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FG_E_ARG, "x, w_qkv, q, k and v must be 16-byte aligned");
  if (Nq % 128 || Nkv % 128 || K % 64)
    return fail(FG_E_UNSUPPORTED,
                "the GEMM tiles need Nq and Nkv multiples of 128 and K %% 64 == 0 "
                "(Nq=%d, Nkv=%d, K=%d)", Nq, Nkv, K);
  const int64_t N64 = (int64_t)Nq + 2 * (int64_t)Nkv;
  if (N64 > INT32_MAX / 2 || (int64_t)T * (N64 / 128) > INT32_MAX)
    return fail(FG_E_UNSUPPORTED, "too many tiles");
  const int N = (int)N64;
  OutSeg o;
  o.y[0] = (u16 *)q;
  o.y[1] = (u16 *)k;
  o.y[2] = (u16 *)v;
  o.col0[0] = 0;
  o.col0[1] = Nq;
  o.col0[2] = Nq + Nkv;
  o.col0[3] = N;
  return run_linear((const u16 *)x, (const u16 *)w_qkv, o, T, K, N, Nq % 256 == 0 && Nkv % 256 == 0,
                    reinterpret_cast<hipStream_t>(stream));
}
