// Sparse decode attention over resolved rows, gfx950.
//
// Each query attends to exactly its k selected rows, in selection order, read from the pool at the
// locations the resolver emitted ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
// Hierarchy", Eq. 1 and section 3.5: placement changes where rows live, not what attention reads).
//
// MLA (DeepSeek-style latent rows): one 576-wide bf16 row per selected position serves as key
// (row[0:dk]) and value (row[0:dv]) for every head.  GQA (Quest-style pages): each selected page row holds
// page_tokens tokens of [K dh | V dh]; query head h reads KV head h / (H / Hkv).
//
// Both use split-k: the k rows of a query are cut into `split` partitions processed by different
// workgroups, each producing a running max m, a running sum l and an unnormalised output o in fp32; a
// combine kernel merges the partitions (o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s) and rounds to
// bf16 (round to nearest even).
#include <cmath>
#include <mutex>
#include <type_traits>
#include <utility>

#include "hsk_internal.h"

namespace hsk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// two floats to a bf16 pair (round to nearest even, v_cvt_pk_bf16_f32), x in the low half
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, v);
}

struct AttnArgs {
  const uint16_t* q;
  const char* pool;
  const int32_t* locs;
  const int32_t* nq;
  uint16_t* out;
  uint16_t* po;  // [RQ][split][H][dv] bf16 partial outputs, each normalised by its own sum
  float* pm;     // [RQ][split][H] partial maxima (natural-log units)
  float* pl;     // [RQ][split][H] partial sums of e^(s - m)
  int32_t R, Qmax, H, Hkv, dk, dv, k, row_elems, page_tokens, split, rows_per_split;
  float scale;
};

// ------------------------------------------------------------------------------------------------------
// MLA on the matrix cores.
//
// One workgroup = NPAIR pairs of waves; pair p owns 16*NHB query heads, and its two waves split the work
// in half: wave `half` computes the partial scores over key dims [288*half, 288*half + 288) and, after the
// pair has summed its partials through LDS, accumulates the output columns [256*half, 256*half + 256).
// Per tile of 32 selected rows:
//   S^T (32 rows x heads) = K (32 x 576) . Q^T            v_mfma_f32_16x16x32_bf16, A = K from LDS,
//                                                          B = Q held in registers for the whole kernel
//   online softmax per head (fp32, exp2 domain)
//   O^T (cols x heads) += V^T (cols x 32 rows) . P        A = V read with ds_read_b64_tr_b16 (transposing
//                                                          loads from the row-major tile), B = P as bf16
// The scores' accumulator layout (lane: head = lane % 16, rows 4*(lane/16)+v of each 16-row block) is used
// directly as the B operand of the P.V product: the 8 rows a lane holds are its k-slots, and the V operand
// is read with the same row order, so no shuffle is needed between the two products.
//
// Rows are gathered by their locations straight from the pool into LDS with 16-byte LDS-DMA loads, three
// tiles in flight.  A tile is stored as 9 groups of 8 chunks (16 bytes each) per row, and the chunk position
// inside a row's 128-byte group is XOR-swizzled by f(a) = ((a & 3) << 1) | (a >> 2), a = (row / 2) mod 8:
// f is a bijection (16-row A-operand reads hit 16 distinct 16-byte bank groups) and f(a) / 2 takes four
// different values on each run of four a (the transposing V reads of 32 lanes, 8 rows x 4 column chunks,
// hit 32 distinct 8-byte bank pairs).
// ------------------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define HSK_LDS __attribute__((address_space(3)))

constexpr int kMlaDk = 576;
constexpr int kMlaDv = 512;
constexpr int kTile = 32;
constexpr int kTileBytes = kTile * kMlaDk * 2;   // 36,864
constexpr int kDmaPerTile = kTileBytes / 1024;   // 36 wave-wide 16-byte loads
constexpr int kBufs = 3;
constexpr int kMaxSplitRows = 2048;
constexpr int kMaxFusedRows = 1024;  // rows per partition of the fused kernel (two location arrays in LDS)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct MlaArgs {
  const uint16_t* q;
  const char* pool;
  const int32_t* locs;
  const int32_t* nq;
  uint16_t* out;
  uint16_t* po;
  float* pm;
  float* pl;
  const int32_t* fill;  // fused resolve + attend: per-selection host source (-1 resident, else 2 p + first)
  const char* host;     // fused: device-visible pinned host rows of request 0 of the source
  int64_t host_req_stride;
  int32_t Qmax, H, k, row_bytes, split, rows_per_split;
  int32_t hgroups, RQ;
  int32_t xcd_groups;  // > 0: the split x hgroups workgroups of one query share an XCD (see mla_block)
  float scale_log2;    // softmax scale * log2(e)
};

// byte offset in a tile of 16-byte chunk c (values 8c..8c+7) of tile row t
__device__ __forceinline__ int tile_swz(int t) {
  const int a = (t >> 1) & 7;
  return ((a & 3) << 1) | (a >> 2);
}
__device__ __forceinline__ int tile_off(int t, int c) {
  const int f = tile_swz(t);
  return (((c >> 3) << 8) + (t << 3) + ((c & 7) ^ f)) << 4;
}

// The LDS-DMA loads are issued from inline assembly so that the compiler, which cannot tell the tile
// buffers apart, does not wait for every load in flight before each LDS read; the kernel waits itself:
// `vmcnt(N)` with N = this wave's loads of the next tile, then a workgroup barrier.
__device__ __forceinline__ void dma16(const char* gsrc, const HSK_LDS char* ldst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)ldst;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(gsrc) : "memory", "m0");
}

// max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows), without LDS: permlane32_swap
// pairs each lane with lane ^ 32, permlane16_swap with lane ^ 16
__device__ __forceinline__ float max_across_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int N>
__device__ __forceinline__ void wait_tile_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_tile_barrier_n(int n) {
  switch (n) {
    case 4: wait_tile_barrier<4>(); break;
    case 5: wait_tile_barrier<5>(); break;
    case 9: wait_tile_barrier<9>(); break;
    case 18: wait_tile_barrier<18>(); break;
    default: wait_tile_barrier<0>(); break;
  }
}

// f(integral_constant<int, U>) for every U of the sequence, in order (compile-time indices for instruction fields)
template <typename F, int... U>
__device__ __forceinline__ void for_each_const(F&& f, std::integer_sequence<int, U...>) {
  (f(std::integral_constant<int, U>{}), ...);
}

// the 32-head kernels' waits: this wave's loads of 0 to 3 tiles (9 or 18 each) still in flight
__device__ __forceinline__ void wait_tile_barrier32(int n) {
  switch (n) {
    case 9: wait_tile_barrier<9>(); break;
    case 18: wait_tile_barrier<18>(); break;
    case 27: wait_tile_barrier<27>(); break;
    case 36: wait_tile_barrier<36>(); break;
    default: wait_tile_barrier<0>(); break;
  }
}

// LDS writes of this wave complete, then a workgroup barrier (no wait on global loads)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// FUSED: rows fetched from host in this call are read straight from pinned host memory (PCIe, zero copy)
// and the first occurrence of each is written from the LDS tile into its pool row; the kernel is then
// bound by the host link, so it waits for each tile's loads one tile ahead only (stores share the in-order
// memory counter with the loads, which rules out the deeper fixed-count waits).
// Workgroup id -> (partition, head group, query).  Workgroups are handed to the 8 XCDs in turn (id mod 8),
// and each XCD has its own L2: with xcd_groups = G > 0 the G = split x hgroups workgroups of query rq get
// ids 8 (G (rq / 8) + g) + rq mod 8, all on one XCD and dispatched together, so the query's Q block (read by
// every partition) and, across head groups, its rows come from that L2 after the first read.  Ids past the
// last query exit at once.  xcd_groups = 0 keeps the plain order (few queries: spreading them over the
// XCDs matters more).
__device__ __forceinline__ bool mla_block(const MlaArgs& a, int id, int* sp, int* hgrp, int* rq) {
  int g, q;
  if (a.xcd_groups > 0) {
    const int x = id & 7, j = id >> 3;
    g = j % a.xcd_groups;
    q = (j / a.xcd_groups) * 8 + x;
  } else {
    g = id % (a.split * a.hgroups);
    q = id / (a.split * a.hgroups);
  }
  *sp = g % a.split;
  *hgrp = g / a.split;
  *rq = q;
  return q < a.RQ;
}

template <int NHB, int NPAIR, bool FUSED>
__global__ __launch_bounds__(128 * NPAIR) void mla_mfma_kernel(MlaArgs a) {
  constexpr int NW = 2 * NPAIR;
  constexpr int NT = 64 * NW;
  constexpr int HW = 16 * NHB;          // heads of one wave pair
  constexpr int KS = kMlaDk / 2 / 32;   // 9 k-steps per half of the key dims
  constexpr int CB = kMlaDv / 2 / 16;   // 16 column blocks per half of the value dims
  constexpr int kGroup = 2048;          // half the bytes of one 8-chunk group of the 32 tile rows
  __shared__ __attribute__((aligned(1024))) char s_tile[kBufs][kTileBytes];
  __shared__ f32x4 s_x[NW][2 * NHB][64];
  __shared__ int32_t s_loc[FUSED ? kMaxFusedRows : kMaxSplitRows];
  __shared__ int32_t s_fill[FUSED ? kMaxFusedRows : 1];

  int sp, hgrp, rq;
  if (!mla_block(a, blockIdx.x, &sp, &hgrp, &rq)) return;
  if (a.nq) {
    const int r = rq / a.Qmax, qi = rq % a.Qmax;
    if (qi >= a.nq[r]) return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1, half = wave & 1;
  const int g = lane >> 4, jl = lane & 15;
  const int i0 = sp * a.rows_per_split;
  const int nrows = max(0, min(a.k, i0 + a.rows_per_split) - i0);
  const int ntiles = (nrows + kTile - 1) / kTile;
  const int hbase = hgrp * (HW * NPAIR) + pair * HW;
  // Tile loads: NWD waves issue them, dw is this wave's index among them (negative: none).  The fused kernel
  // with eight waves gives them to waves 4-7 and its pool write-backs to waves 0-1, so the loading waves'
  // memory counter counts only loads and two tiles can be in flight, as in the plain kernel.
  constexpr bool kSplitRoles = FUSED && NW == 8;
  constexpr int NWD = kSplitRoles ? 4 : NW;
  const int dw = kSplitRoles ? wave - 4 : wave;
  const int my_dma = dw < 0 ? 0 : (kDmaPerTile - dw + NWD - 1) / NWD;

  // a negative location (every location of a request the resolve rejected is -1) reads row 0: such a
  // query's output is meaningless, but no load leaves the pool
  const int32_t* locs = a.locs + (int64_t)rq * a.k + i0;
  for (int x = tid; x < nrows; x += NT) {
    s_loc[x] = max(locs[x], 0);
    if constexpr (FUSED) s_fill[x] = a.fill[(int64_t)rq * a.k + i0 + x];
  }
  const char* hostr = FUSED ? a.host + (int64_t)(rq / a.Qmax) * a.host_req_stride : nullptr;

  bf16x8 qf[NHB][KS];
  {
    const uint16_t* qb = a.q + ((int64_t)rq * a.H + hbase + jl) * kMlaDk + 288 * half + 8 * g;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[hb][ks] = *(const bf16x8*)(qb + (int64_t)hb * 16 * kMlaDk + 32 * ks);
  }
  // Q and the locations are in registers/LDS before any tile load is issued: the compiler then has no
  // global load of its own in flight inside the loop, where a vmcnt wait would also wait for the tiles.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Lane-constant parts of the LDS addresses; every unrolled read adds a compile-time offset.
  //  S:  chunk 36 half + 4 ks + g of row 16 tb + jl.  Even and odd ks differ in the swizzled position;
  //      ks and ks + 2 are one 4,096-byte chunk group apart; tb = 1 is 2,048 bytes after tb = 0.
  const int s_even = tile_off(jl, 36 * half + g);
  const int s_odd = tile_off(jl, 36 * half + g + 4);
  //  PV: chunk 32 half + 2 cb + (q4 >> 1) of row t1 (and t1 + 16), byte (q4 & 1) * 8; cb = 4 u + w.
  const int t1 = 4 * g + (jl >> 2);
  const int q4 = jl & 3;
  int v_base[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) v_base[w] = tile_off(t1, 32 * half + 2 * w + (q4 >> 1)) + (q4 & 1) * 8;
  // DMA: wave-wide load i (i = dw + NWD u) covers tile rows 8 (i & 3) .. + 7 and chunk group i >> 2; a
  // lane copies 16 bytes of one row: with 4 or more loading waves every load of a wave uses the same rows
  // (NTOK = 1), with 2 the loads alternate between two rows.
  constexpr int NTOK = NWD >= 4 ? 1 : 2;
  const uint32_t lds_tile0 = (uint32_t)(uintptr_t)(const HSK_LDS char*)&s_tile[0][0];
  auto issue = [&](int T, int b) {
    const int tb = T * kTile;
    const uint32_t lbase = lds_tile0 + b * kTileBytes + dw * 1024;
    // the row and lane offset are recomputed from the lane id at every issue (a few VALU operations) rather
    // than kept live across the loop, where registers are short
    // (volatile, so that the compiler cannot hoist it and its uses out of the loop again)
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const char* rp[NTOK];
#pragma unroll
    for (int v = 0; v < NTOK; ++v) {
      const int tok = 8 * ((dw + NWD * v) & 3) + (ln >> 3);
      const int sw = (((ln & 7) ^ tile_swz(tok)) << 4) + (NWD >= 4 ? (dw >> 2) * 128 : 0);
      const int x = tb + tok < nrows ? tb + tok : 0;   // rows past the end re-read row 0 (masked)
      const int32_t loc = s_loc[x];
      if (FUSED && s_fill[x] >= 0) {
        rp[v] = hostr + ((int64_t)(s_fill[x] >> 1) * a.row_bytes + sw);
      } else {
        // the locations of a request the resolve rejected are -1: the fused kernel reads row 0 for them
        rp[v] = a.pool + ((int64_t)(FUSED && loc < 0 ? 0 : loc) * a.row_bytes + sw);
      }
    }
#pragma unroll
    for (int u = 0; u < (kDmaPerTile + NWD - 1) / NWD; ++u) {
      if (dw + NWD * u < kDmaPerTile) {
        // the instruction's immediate offset would also move the LDS destination, so the row offset of
        // the chunk group goes into the address register
        constexpr int kStep = NWD >= 4 ? (NWD / 4) * 128 : 0;
        const uint32_t m0 = lbase + NWD * u * 1024;
        const char* src = NWD >= 4 ? rp[0] + kStep * u : rp[u % NTOK] + (u >> 1) * 128;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
      }
    }
  };

  f32x4 oacc[CB][NHB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) oacc[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NHB], l_run[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) { m_run[hb] = -INFINITY; l_run[hb] = 0.f; }

  // Tile phases.  score_phase(T): this wave's partial scores over its half of the key dims, written to
  // s_x for the partner.  pv_phase(T): the partner's partials (visible after a barrier) completed into
  // scores, online softmax, then O += P V over this wave's half of the value columns.
  f32x4 sacc[2][NHB];
  auto score_phase = [&](int T) {
    const HSK_LDS char* tile = (const HSK_LDS char*)&s_tile[T % kBufs][0];
    // partial scores over this wave's half of the key dims
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sacc[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const HSK_LDS char* se = tile + s_even;
    const HSK_LDS char* so = tile + s_odd;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const HSK_LDS char* sb = (ks & 1) ? so + (ks >> 1) * kGroup * 2 : se + (ks >> 1) * kGroup * 2;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 kf = *(const HSK_LDS bf16x8*)(sb + tb * 2048);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
          sacc[tb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[hb][ks], sacc[tb][hb], 0, 0, 0);
      }
    }
    // the pair sums its two halves (both waves get the same, commutative, sum)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) s_x[wave][tb * NHB + hb][lane] = sacc[tb][hb];
  };
  auto pv_phase = [&](int T) {
    const HSK_LDS char* tile = (const HSK_LDS char*)&s_tile[T % kBufs][0];
    const int rem = nrows - T * kTile;
    // the partner's partial blocks complete the scores
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sacc[tb][hb] += s_x[wave ^ 1][tb * NHB + hb][lane];

    // online softmax; lane holds head hbase + 16 hb + jl, rows 16 tb + 4 g + v.  The maximum is taken over
    // the unscaled scores (the scale is positive) and the scale is applied inside the exponent's FMA;
    // only the last tile of a partition masks rows.
    const bool full = rem >= kTile;
    bf16x8 pf[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float sv[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[4 * tb + v] = sacc[tb][hb][v];
      if (!full) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (16 * (i >> 2) + 4 * g + (i & 3) >= rem) sv[i] = -INFINITY;
      }
      float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      tmax = max_across_row_groups(tmax) * a.scale_log2;
      // The reference maximum moves only when a score exceeds it by more than 2^8 (log2 units 8): until
      // then the weights exp2(s - m) stay below 256, exact enough in bf16 and fp32, and the 128 output
      // accumulators need no rescaling.  The first tile always moves it (from -inf).
      if (__ballot(tmax > m_run[hb] + 8.f)) {
        const float mn = fmaxf(m_run[hb], tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run[hb] - mn);
        l_run[hb] *= alpha;
        m_run[hb] = mn;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) oacc[cb][hb] *= alpha;
      }
      const float mneg = -m_run[hb];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sv[i], a.scale_log2, mneg));
        psum += p;
        pf[hb][i] = (__bf16)p;
      }
      l_run[hb] += psum;
    }

    // O^T += V^T P over this wave's half of the value columns.  The transposing reads are issued from
    // inline assembly with immediate offsets from four per-tile base addresses (column block cb = 4 u + w
    // reads base w + u * 4096, rows 16..31 2048 bytes further), two column blocks ahead of their products.
    {
      const uint32_t tb0 = (uint32_t)(uintptr_t)tile;
      const uint32_t vb0 = tb0 + v_base[0], vb1 = tb0 + v_base[1], vb2 = tb0 + v_base[2], vb3 = tb0 + v_base[3];
      i16x4 vlo[3], vhi[3];
#define HSK_TR_READ(CB)                                                                                   \
  {                                                                                                      \
    const uint32_t vb_ = ((CB)&3) == 0 ? vb0 : ((CB)&3) == 1 ? vb1 : ((CB)&3) == 2 ? vb2 : vb3;        \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"                                                   \
                 : "=v"(vlo[(CB) % 3]) : "v"(vb_), "i"(((CB) >> 2) * 4096) : "memory");                 \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"                                                   \
                 : "=v"(vhi[(CB) % 3]) : "v"(vb_), "i"(((CB) >> 2) * 4096 + 2048) : "memory");          \
  }
#define HSK_PV_STEP(CB, WAIT)                                                                             \
  {                                                                                                      \
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(vlo[(CB) % 3]), "+v"(vhi[(CB) % 3]) : "i"(WAIT));      \
    const bf16x8 vf = __builtin_bit_cast(                                                                \
        bf16x8, __builtin_shufflevector(vlo[(CB) % 3], vhi[(CB) % 3], 0, 1, 2, 3, 4, 5, 6, 7));         \
    _Pragma("unroll") for (int hb = 0; hb < NHB; ++hb) oacc[CB][hb] =                                   \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[hb], oacc[CB][hb], 0, 0, 0);                     \
  }
      HSK_TR_READ(0) HSK_TR_READ(1)
      HSK_TR_READ(2) HSK_PV_STEP(0, 4)
      HSK_TR_READ(3) HSK_PV_STEP(1, 4)
      HSK_TR_READ(4) HSK_PV_STEP(2, 4)
      HSK_TR_READ(5) HSK_PV_STEP(3, 4)
      HSK_TR_READ(6) HSK_PV_STEP(4, 4)
      HSK_TR_READ(7) HSK_PV_STEP(5, 4)
      HSK_TR_READ(8) HSK_PV_STEP(6, 4)
      HSK_TR_READ(9) HSK_PV_STEP(7, 4)
      HSK_TR_READ(10) HSK_PV_STEP(8, 4)
      HSK_TR_READ(11) HSK_PV_STEP(9, 4)
      HSK_TR_READ(12) HSK_PV_STEP(10, 4)
      HSK_TR_READ(13) HSK_PV_STEP(11, 4)
      HSK_TR_READ(14) HSK_PV_STEP(12, 4)
      HSK_TR_READ(15) HSK_PV_STEP(13, 4)
      HSK_PV_STEP(14, 2)
      HSK_PV_STEP(15, 0)
#undef HSK_TR_READ
#undef HSK_PV_STEP
      static_assert(CB == 16, "the unrolled P.V sequence covers 16 column blocks");
    }
  };

  if (dw >= 0) {
    if (ntiles > 0) issue(0, 0);
    if ((!FUSED || kSplitRoles) && ntiles > 1) issue(1, 1);
  }
  for (int T = 0; T < ntiles; ++T) {
    if (kSplitRoles) {
      // loading waves wait for their loads of tile T (tile T + 1 may stay in flight); the others have only
      // stores outstanding and need not wait for them
      if (dw >= 0) {
        if (T + 1 < ntiles) wait_tile_barrier_n(my_dma); else wait_tile_barrier<0>();
        if (T + 2 < ntiles) issue(T + 2, (T + 2) % kBufs);
      } else {
        lds_barrier();
      }
    } else if (FUSED) {
      wait_tile_barrier<0>();
      if (T + 1 < ntiles) issue(T + 1, (T + 1) % kBufs);
    } else {
      if (T + 1 < ntiles) wait_tile_barrier_n(my_dma); else wait_tile_barrier<0>();
      if (T + 2 < ntiles) issue(T + 2, (T + 2) % kBufs);
    }
    if constexpr (FUSED) {
      const HSK_LDS char* tile = (const HSK_LDS char*)&s_tile[T % kBufs][0];
      const int rem = nrows - T * kTile;
      // the rows this call fetched for the first time go from the tile into their pool rows
      uint32_t wb;
      {
        const int x = T * kTile + (lane & 31);
        wb = (uint32_t)__ballot(hgrp == 0 && (lane & 31) < rem && (s_fill[x < nrows ? x : 0] & 1));
      }
      for (uint32_t mm = wb; mm; mm &= mm - 1) {
        const int row = __builtin_ctz(mm);
        if (tid < kMlaDk / 8) {
          const u32x4 v = *(const HSK_LDS u32x4*)(tile + tile_off(row, tid));
          *(u32x4*)(a.pool + (int64_t)s_loc[T * kTile + row] * a.row_bytes + tid * 16) = v;
        }
      }
    }
    score_phase(T);
    lds_barrier();
    pv_phase(T);
  }

  // epilogue: lane holds head hbase + 16 hb + jl, columns 256 half + 16 cb + 4 g + v
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float l = l_run[hb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int head = hbase + 16 * hb + jl;
    // the output (one partition) or the partition's output normalised by its own sum, in bf16
    const float inv = 1.f / l;
    const int64_t ps = ((int64_t)rq * a.split + sp) * a.H + head;
    uint16_t* o = (a.split == 1 ? a.out + ((int64_t)rq * a.H + head) * kMlaDv : a.po + ps * kMlaDv) +
                  256 * half + 4 * g;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const f32x4 v = oacc[cb][hb] * inv;
      u32x2 w;
      w.x = pack_bf16(v[0], v[1]);
      w.y = pack_bf16(v[2], v[3]);
      *(u32x2*)(o + 16 * cb) = w;
    }
    if (a.split > 1 && half == 0 && g == 0) {
      a.pm[ps] = m_run[hb] * kLn2;   // natural-log units, as the combine expects
      a.pl[ps] = l;
    }
  }
}

// ------------------------------------------------------------------------------------------------------
// MLA with one wave per SIMD and 32 heads per wave (v_mfma_f32_32x32x16_bf16).
//
// Each wave holds the query block of its 32 heads over the whole key width (36 16-dim chunks, 144
// registers) and accumulates its 32 heads' output over all 512 value columns (256 accumulators), so the
// waves of a workgroup never exchange scores and a tile needs one workgroup barrier (the one that lets a
// tile buffer be refilled).  Per tile of 32 selected rows and wave:
//   S^T (32 rows x 32 heads) = K (32 x 576) . Q^T        36 products, A = K from LDS (16-byte reads:
//                                                       lane l reads row l % 32, dims 8 (l / 32) .. + 7
//                                                       of each 16-dim chunk), B = Q in registers
//   online softmax per head (fp32, exp2 domain)
//   O^T (512 cols x 32 heads) += V^T . P                 32 products, A = V through transposing reads,
//                                                       B = P as bf16
// The scores' accumulator layout (lane l: head l % 32, rows 8 (v / 4) + 4 (l / 32) + v % 4 of element v)
// is used as-is for the B operand of P.V: a lane's elements 8 ch .. 8 ch + 7 are its k-slots of the 16-row
// chunk ch, and the transposing reads fetch V in the same row order (rows 16 ch + 8 p + 4 (l / 32) + 0..3
// for part p), so no data moves between lanes between the two products.
// Tiles use the chunk swizzle g(a) = ((a & 1) << 2) | (a >> 1), a = (row / 2) mod 8: g is a bijection (the
// 16 rows of a K read hit 16 distinct 16-byte bank groups) and rows 4m and 4m + 2 get different bit 2 (the
// 32 lanes of a transposing read, 4 rows x 64 bytes, hit 64 distinct banks).  Four tile buffers keep
// three tiles in flight.
// ------------------------------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kBufs32 = 4;

__device__ __forceinline__ int tile_swz32(int t) {
  const int a = (t >> 1) & 7;
  return ((a & 1) << 2) | (a >> 1);
}
__device__ __forceinline__ int tile_off32(int t, int c) {
  return (((c >> 3) << 8) + (t << 3) + ((c & 7) ^ tile_swz32(t))) << 4;
}

template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla32_kernel(MlaArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int KC = kMlaDk / 16;              // 36 16-dim chunks of the key
  constexpr int CB = kMlaDv / 32;              // 16 blocks of 32 value columns
  constexpr int MY = kDmaPerTile / NW;         // this wave's tile loads
  static_assert(kDmaPerTile % NW == 0 && (NW == 2 || NW == 4), "four or two waves");
  __shared__ __attribute__((aligned(1024))) char s_tile[kBufs32][kTileBytes];
  __shared__ int32_t s_loc[kMaxSplitRows];

  int sp, hgrp, rq;
  if (!mla_block(a, blockIdx.x, &sp, &hgrp, &rq)) return;
  if (a.nq) {
    const int r = rq / a.Qmax, qi = rq % a.Qmax;
    if (qi >= a.nq[r]) return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, j = lane & 31;
  const int i0 = sp * a.rows_per_split;
  const int nrows = max(0, min(a.k, i0 + a.rows_per_split) - i0);
  const int ntiles = (nrows + kTile - 1) / kTile;
  const int hbase = hgrp * (32 * NW) + wave * 32;

  const int32_t* locs = a.locs + (int64_t)rq * a.k + i0;
  // negative locations (a request the resolve rejected) read row 0: meaningless output, no load outside the pool
  for (int x = tid; x < nrows; x += NT) s_loc[x] = max(locs[x], 0);
  __syncthreads();
  // The query block is requested first, then the first tiles: loads of a wave complete in order, so the
  // first score products (which wait for the query chunks as the compiler counts them, i.e. for
  // everything issued before each chunk) wait for the query block and only as much of the tiles as
  // precedes each chunk's turn, instead of for all three tiles.
  bf16x8 qf[KC];

  // LDS offsets.  K: row j, chunk 2c + h; for c = 4 u + w that is chunk group u (4,096 bytes further per u)
  // at the position of chunk 2 w + h.  V: part p of chunk ch, column block cb: row 16 ch + 8 p + 4 h + (i >> 2)
  // and 16-byte chunk 4 cb + 2 ((lane >> 4) & 1) + ((i & 3) >> 1), byte (i & 1) * 8, i = lane & 15; column
  // blocks 2 u and 2 u + 1 are chunk group u at positions 0-3 and 4-7.
  int kb[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) kb[w] = tile_off32(j, 2 * w + h);
  int vb[2][2][2];
  {
    const int i = lane & 15, x = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int row = 16 * ch + 8 * p + 4 * h + (i >> 2);
#pragma unroll
        for (int o = 0; o < 2; ++o) vb[ch][p][o] = tile_off32(row, 4 * o + x) + (i & 1) * 8;
      }
  }
  // DMA: wave-wide load i (i = wave + NW u) covers tile rows 8 (i & 3) .. + 7 of chunk group i >> 2; a lane
  // copies 16 bytes of one row (four waves: always the same row; two waves: two rows in turn).
  constexpr int NTOK = NW >= 4 ? 1 : 2;
  const uint32_t lds_tile0 = (uint32_t)(uintptr_t)(const HSK_LDS char*)&s_tile[0][0];
  auto issue = [&](int T, int b) {
    const int tb = T * kTile;
    const uint32_t lbase = lds_tile0 + b * kTileBytes + wave * 1024;
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const char* rp[NTOK];
#pragma unroll
    for (int v = 0; v < NTOK; ++v) {
      const int tok = 8 * ((wave + NW * v) & 3) + (ln >> 3);
      const int sw = ((ln & 7) ^ tile_swz32(tok)) << 4;
      const int x = tb + tok < nrows ? tb + tok : 0;   // rows past the end re-read row 0 (masked)
      rp[v] = a.pool + ((int64_t)s_loc[x] * a.row_bytes + sw);
    }
    const char* const r0 = rp[0];
    const char* const r1 = rp[NTOK - 1];
    auto one = [lbase, r0, r1](auto u_c) {
      constexpr int u = decltype(u_c)::value;
      constexpr int off = (NW >= 4 ? u : u >> 1) * 128;
      // the instruction offset moves the LDS destination as well as the global address: M0 takes it back
      const uint32_t m0 = lbase + NW * u * 1024 - off;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
                   ::"s"(m0), "v"(NW >= 4 || u % 2 == 0 ? r0 : r1), "i"(off) : "memory", "m0");
    };
    for_each_const(one, std::make_integer_sequence<int, MY>{});
  };
  {
    const uint16_t* qb = a.q + ((int64_t)rq * a.H + hbase + j) * kMlaDk + 8 * h;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = *(const bf16x8*)(qb + 16 * c);
  }
#pragma unroll
  for (int T = 0; T < kBufs32 - 1; ++T)
    if (T < ntiles) issue(T, T);
  // The scores of a wave's head are weighed against one reference maximum m_ref, the maximum of the
  // partition's first tile, and the output is never rescaled inside the loop (rescaling 256 accumulators
  // held in the accumulation registers costs more than the loop can afford).  exp2(s - m_ref) stays below
  // 2^64 as long as no later score exceeds m_ref by more than 64 (log2 units); if one does, the workgroup
  // redoes the partition: a pass over the tiles for the true maximum, then the full pass against it.
  f32x16 oacc[CB];
  float m_ref = 0.f, l_run = 0.f;
  // S of tile T for this wave's 32 heads.  The K reads are issued from inline assembly two chunks ahead of
  // their products, with the waits written out (LDS reads of one wave complete in order), from four base
  // registers per tile and immediate offsets.
  // The score products are written in assembly too, in the form that accumulates in ordinary VGPRs: the 256
  // output accumulators fill the accumulation registers, and a builtin product would put S there as well
  // (272 of 256), so that the compiler moved one output block and S between the two files on every tile.
  // Their hazards, which the compiler does not see in assembly: a chain's products accumulate into the same
  // registers (no wait states needed); the first takes 0 for the accumulator; the last is followed by 20 wait
  // states before anything may read S; the operands come from LDS reads (waited for) and from the query
  // block loaded before the loop, never from a VALU write just before a product.
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  auto scores = [&](const HSK_LDS char* tile, auto&& side) {
    const uint32_t t0 = (uint32_t)(uintptr_t)tile;
    const uint32_t kb0 = t0 + kb[0], kb1 = t0 + kb[1], kb2 = t0 + kb[2], kb3 = t0 + kb[3];
    u32x4v kf[3];
    f32x16 sc, out;
#define HSK_K_READ(C)                                                                                       \
  {                                                                                                        \
    const uint32_t b_ = ((C)&3) == 0 ? kb0 : ((C)&3) == 1 ? kb1 : ((C)&3) == 2 ? kb2 : kb3;               \
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[(C) % 3]) : "v"(b_), "i"(((C) >> 2) * 4096) : "memory"); \
  }
#define HSK_K_STEP(C, WAIT)                                                                                 \
  {                                                                                                        \
    if ((C) == 0)                                                                                          \
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"                       \
                   : "=&v"(sc) : "v"(kf[0]), "v"(qf[0]), "i"(WAIT));                                       \
    else if ((C) < KC - 1)                                                                                 \
      asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"                      \
                   : "+v"(sc) : "v"(kf[(C) % 3]), "v"(qf[C]), "i"(WAIT));                                  \
    else                                                                                                   \
      asm volatile("s_waitcnt lgkmcnt(%4)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3" \
                   : "=&v"(out) : "v"(kf[(C) % 3]), "v"(qf[C]), "v"(sc), "i"(WAIT));                       \
  }
    HSK_K_READ(0) HSK_K_READ(1)
    HSK_K_READ(2) HSK_K_STEP(0, 2) side(std::integral_constant<int, 0>{});
    HSK_K_READ(3) HSK_K_STEP(1, 2) side(std::integral_constant<int, 1>{});
    HSK_K_READ(4) HSK_K_STEP(2, 2) side(std::integral_constant<int, 2>{});
    HSK_K_READ(5) HSK_K_STEP(3, 2) side(std::integral_constant<int, 3>{});
    HSK_K_READ(6) HSK_K_STEP(4, 2) side(std::integral_constant<int, 4>{});
    HSK_K_READ(7) HSK_K_STEP(5, 2) side(std::integral_constant<int, 5>{});
    HSK_K_READ(8) HSK_K_STEP(6, 2) side(std::integral_constant<int, 6>{});
    HSK_K_READ(9) HSK_K_STEP(7, 2) side(std::integral_constant<int, 7>{});
    HSK_K_READ(10) HSK_K_STEP(8, 2) side(std::integral_constant<int, 8>{});
    HSK_K_READ(11) HSK_K_STEP(9, 2) side(std::integral_constant<int, 9>{});
    HSK_K_READ(12) HSK_K_STEP(10, 2) side(std::integral_constant<int, 10>{});
    HSK_K_READ(13) HSK_K_STEP(11, 2) side(std::integral_constant<int, 11>{});
    HSK_K_READ(14) HSK_K_STEP(12, 2) side(std::integral_constant<int, 12>{});
    HSK_K_READ(15) HSK_K_STEP(13, 2) side(std::integral_constant<int, 13>{});
    HSK_K_READ(16) HSK_K_STEP(14, 2) side(std::integral_constant<int, 14>{});
    HSK_K_READ(17) HSK_K_STEP(15, 2) side(std::integral_constant<int, 15>{});
    HSK_K_READ(18) HSK_K_STEP(16, 2) side(std::integral_constant<int, 16>{});
    HSK_K_READ(19) HSK_K_STEP(17, 2) side(std::integral_constant<int, 17>{});
    HSK_K_READ(20) HSK_K_STEP(18, 2) side(std::integral_constant<int, 18>{});
    HSK_K_READ(21) HSK_K_STEP(19, 2) side(std::integral_constant<int, 19>{});
    HSK_K_READ(22) HSK_K_STEP(20, 2) side(std::integral_constant<int, 20>{});
    HSK_K_READ(23) HSK_K_STEP(21, 2) side(std::integral_constant<int, 21>{});
    HSK_K_READ(24) HSK_K_STEP(22, 2) side(std::integral_constant<int, 22>{});
    HSK_K_READ(25) HSK_K_STEP(23, 2) side(std::integral_constant<int, 23>{});
    HSK_K_READ(26) HSK_K_STEP(24, 2) side(std::integral_constant<int, 24>{});
    HSK_K_READ(27) HSK_K_STEP(25, 2) side(std::integral_constant<int, 25>{});
    HSK_K_READ(28) HSK_K_STEP(26, 2) side(std::integral_constant<int, 26>{});
    HSK_K_READ(29) HSK_K_STEP(27, 2) side(std::integral_constant<int, 27>{});
    HSK_K_READ(30) HSK_K_STEP(28, 2) side(std::integral_constant<int, 28>{});
    HSK_K_READ(31) HSK_K_STEP(29, 2) side(std::integral_constant<int, 29>{});
    HSK_K_READ(32) HSK_K_STEP(30, 2) side(std::integral_constant<int, 30>{});
    HSK_K_READ(33) HSK_K_STEP(31, 2) side(std::integral_constant<int, 31>{});
    HSK_K_READ(34) HSK_K_STEP(32, 2) side(std::integral_constant<int, 32>{});
    HSK_K_READ(35) HSK_K_STEP(33, 2) side(std::integral_constant<int, 33>{});
    HSK_K_STEP(34, 1) side(std::integral_constant<int, 34>{});
    HSK_K_STEP(35, 0) side(std::integral_constant<int, 35>{});
#undef HSK_K_READ
#undef HSK_K_STEP
    static_assert(KC == 36, "the unrolled score sequence covers 36 chunks");
    return out;
  };
  // maximum over the valid rows of a tile, in log2 units, the same in lanes l and l ^ 32 (rows past the
  // partition's end are set to -inf without a branch)
  auto tile_max = [&](f32x16& sc, int T) {
    const int rem = nrows - T * kTile;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 8 * (v >> 2) + 4 * h + (v & 3) < rem ? sc[v] : -INFINITY;
    float tmax = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, sc[v]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
  };
  // softmax weights of tile T against m_ref (set from tile 0 when set_ref), as the bf16 B operands of P.V
  bool over = false;
  auto softmax = [&](f32x16 sc, int T, bool set_ref, bf16x8 (&pf)[2]) {
    const float tmax = tile_max(sc, T);
    m_ref = set_ref && T == 0 ? tmax : m_ref;
    over |= tmax > m_ref + 64.f;
    const float mneg = -m_ref;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sc[v], a.scale_log2, mneg));
      psum += pv;
      pf[v >> 3][v & 7] = (__bf16)pv;
    }
    l_run += psum;
  };
  // O^T += V^T P over one tile: step 2 cb + ch (column block cb, chunk ch) multiplies two transposing reads
  // (parts 0 and 1: 8 rows of V) by P; the reads run two steps ahead, from eight base registers per tile
  auto pv = [&](const HSK_LDS char* tile, const bf16x8 (&pf)[2]) {
    const uint32_t t0 = (uint32_t)(uintptr_t)tile;
    const uint32_t v000 = t0 + vb[0][0][0], v001 = t0 + vb[0][0][1], v010 = t0 + vb[0][1][0],
                   v011 = t0 + vb[0][1][1], v100 = t0 + vb[1][0][0], v101 = t0 + vb[1][0][1],
                   v110 = t0 + vb[1][1][0], v111 = t0 + vb[1][1][1];
    i16x4 vlo[3], vhi[3];
#define HSK_V_READ(S)                                                                                      \
  {                                                                                                       \
    constexpr int cb_ = (S) >> 1, ch_ = (S)&1;                                                            \
    const uint32_t b0_ = ch_ ? ((cb_ & 1) ? v101 : v100) : ((cb_ & 1) ? v001 : v000);                     \
    const uint32_t b1_ = ch_ ? ((cb_ & 1) ? v111 : v110) : ((cb_ & 1) ? v011 : v010);                     \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vlo[(S) % 3]) : "v"(b0_), "i"((cb_ >> 1) * 4096) : "memory"); \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vhi[(S) % 3]) : "v"(b1_), "i"((cb_ >> 1) * 4096) : "memory"); \
  }
#define HSK_V_STEP(S, WAIT)                                                                                \
  {                                                                                                       \
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(vlo[(S) % 3]), "+v"(vhi[(S) % 3]) : "i"(WAIT));           \
    const bf16x8 vf_ = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[(S) % 3], vhi[(S) % 3], 0, 1, 2, 3, 4, 5, 6, 7)); \
    oacc[(S) >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf_, pf[(S)&1], oacc[(S) >> 1], 0, 0, 0);  \
  }
    HSK_V_READ(0) HSK_V_READ(1)
    HSK_V_READ(2) HSK_V_STEP(0, 4)
    HSK_V_READ(3) HSK_V_STEP(1, 4)
    HSK_V_READ(4) HSK_V_STEP(2, 4)
    HSK_V_READ(5) HSK_V_STEP(3, 4)
    HSK_V_READ(6) HSK_V_STEP(4, 4)
    HSK_V_READ(7) HSK_V_STEP(5, 4)
    HSK_V_READ(8) HSK_V_STEP(6, 4)
    HSK_V_READ(9) HSK_V_STEP(7, 4)
    HSK_V_READ(10) HSK_V_STEP(8, 4)
    HSK_V_READ(11) HSK_V_STEP(9, 4)
    HSK_V_READ(12) HSK_V_STEP(10, 4)
    HSK_V_READ(13) HSK_V_STEP(11, 4)
    HSK_V_READ(14) HSK_V_STEP(12, 4)
    HSK_V_READ(15) HSK_V_STEP(13, 4)
    HSK_V_READ(16) HSK_V_STEP(14, 4)
    HSK_V_READ(17) HSK_V_STEP(15, 4)
    HSK_V_READ(18) HSK_V_STEP(16, 4)
    HSK_V_READ(19) HSK_V_STEP(17, 4)
    HSK_V_READ(20) HSK_V_STEP(18, 4)
    HSK_V_READ(21) HSK_V_STEP(19, 4)
    HSK_V_READ(22) HSK_V_STEP(20, 4)
    HSK_V_READ(23) HSK_V_STEP(21, 4)
    HSK_V_READ(24) HSK_V_STEP(22, 4)
    HSK_V_READ(25) HSK_V_STEP(23, 4)
    HSK_V_READ(26) HSK_V_STEP(24, 4)
    HSK_V_READ(27) HSK_V_STEP(25, 4)
    HSK_V_READ(28) HSK_V_STEP(26, 4)
    HSK_V_READ(29) HSK_V_STEP(27, 4)
    HSK_V_READ(30) HSK_V_STEP(28, 4)
    HSK_V_READ(31) HSK_V_STEP(29, 4)
    HSK_V_STEP(30, 2)
    HSK_V_STEP(31, 0)
#undef HSK_V_READ
#undef HSK_V_STEP
    static_assert(CB == 16, "the unrolled P.V sequence covers 32 steps");
  };
  // The full pass is software-pipelined by one tile: iteration T computes S of tile T + 1 and, in the same
  // straight-line block, the softmax and P.V of tile T, so the matrix cores are fed while the softmax of
  // the previous tile runs.  Tile T + 3 is loaded into the buffer of tile T - 1, which every wave has
  // finished with at the barrier that also makes tile T + 1 visible.
  auto no_side = [](auto) {};
  auto full_pass = [&](bool set_ref, bool issued) {
    if (!issued) {
#pragma unroll
      for (int T = 0; T < kBufs32 - 1; ++T)
        if (T < ntiles) issue(T, T);
    }
    // (loads complete in order: this wait for tile 0 also covers the query block read before it, when
    // the first tiles were issued with it)
    wait_tile_barrier32(MY * min(ntiles - 1, kBufs32 - 2));
    f32x16 sc = scores((const HSK_LDS char*)&s_tile[0][0], no_side);
    bf16x8 pf[2];
    for (int T = 0; T + 1 < ntiles; ++T) {
      wait_tile_barrier32(MY * min(ntiles - 2 - T, 1));
      // Tile T + 3 is loaded during S(T + 1), one of this wave's MY loads every kDmaStride products, so that
      // the CU's vector memory path moves the tile while the matrix cores work (issued together before the
      // products, the loads held each wave ~600 cycles per tile).  The LDS read of the lane's source row
      // location(s) is issued first, from inline assembly: the K reads' explicit waits (in-order LDS
      // completion) cover it before its first use at the first load.
      constexpr int kDmaStride = 36 / MY;
      const bool load_next = T + kBufs32 - 1 < ntiles;
      const uint32_t lnext = lds_tile0 + ((T + kBufs32 - 1) % kBufs32) * kTileBytes + wave * 1024;
      int32_t lv[NTOK];
      const char* rp[NTOK];
      if (load_next) {
        const int tb = (T + kBufs32 - 1) * kTile;
#pragma unroll
        for (int v = 0; v < NTOK; ++v) {
          const int tok = 8 * ((wave + NW * v) & 3) + (lane >> 3);
          const int x = tb + tok < nrows ? tb + tok : 0;   // rows past the end re-read row 0 (masked)
          asm volatile("ds_read_b32 %0, %1" : "=v"(lv[v]) : "v"((uint32_t)(uintptr_t)(const HSK_LDS int32_t*)&s_loc[x]) : "memory");
        }
      }
      auto dma_step = [&](auto step_c) {
        constexpr int step = decltype(step_c)::value;
        if constexpr (step % kDmaStride == 1 && step / kDmaStride < MY) {
        if (!load_next) return;
        constexpr int u = step / kDmaStride;
        if constexpr (u == 0) {
          // the location reads went out before the K reads, and after the product just issued at most the two
          // newest K reads are outstanding, so they are complete: this wait (already met) ties their first use
          // here, where the compiler could otherwise move it ahead of the waits it does not see
          if constexpr (NTOK == 1)
            asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(lv[0]));
          else
            asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(lv[0]), "+v"(lv[NTOK - 1]));
#pragma unroll
          for (int v = 0; v < NTOK; ++v) {
            const int tok = 8 * ((wave + NW * v) & 3) + (lane >> 3);
            rp[v] = a.pool + ((int64_t)lv[v] * a.row_bytes + (((lane & 7) ^ tile_swz32(tok)) << 4));
          }
        }
        // the load's chunk group goes into the instruction's offset field (no address arithmetic per load);
        // that offset also moves the LDS destination, which M0 takes back
        constexpr int off = (NW >= 4 ? u : u >> 1) * 128;
        const uint32_t m0 = lnext + NW * u * 1024 - off;
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
                     ::"s"(m0), "v"(rp[NW >= 4 ? 0 : u % NTOK]), "i"(off) : "memory", "m0");
        }
      };
      // the softmax of tile T in six pieces between the products of S(T + 1): masks and maxima, the
      // cross-lane maximum and reference, then the exponentials four at a time and the bf16 packing
      const int rem = nrows - T * kTile;
      float tmx = -INFINITY, mneg = 0.f, psum = 0.f, pw[16];
      auto side = [&](auto step_c) {
        constexpr int step = decltype(step_c)::value;
        dma_step(step_c);
        if ((step & 3) != 3 || step > 23) return;
        const int piece = step >> 2;
        if (piece <= 1) {
          if (rem >= kTile) {   // wave-uniform: only a partition's last tile can hold rows past its end
#pragma unroll
            for (int v = 8 * piece; v < 8 * piece + 8; ++v) tmx = fmaxf(tmx, sc[v]);
          } else {
#pragma unroll
            for (int v = 8 * piece; v < 8 * piece + 8; ++v) {
              sc[v] = 8 * (v >> 2) + 4 * h + (v & 3) < rem ? sc[v] : -INFINITY;
              tmx = fmaxf(tmx, sc[v]);
            }
          }
          if (piece == 1) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmx), __float_as_uint(tmx), false, false);
            const float tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
            m_ref = set_ref && T == 0 ? tmax : m_ref;
            over |= tmax > m_ref + 64.f;
            mneg = -m_ref;
          }
        } else {
#pragma unroll
          for (int v = 4 * (piece - 2); v < 4 * (piece - 2) + 4; ++v) {
            pw[v] = __builtin_amdgcn_exp2f(fmaf(sc[v], a.scale_log2, mneg));
            psum += pw[v];
          }
          if (piece == 5) {
#pragma unroll
            for (int v = 0; v < 16; ++v) pf[v >> 3][v & 7] = (__bf16)pw[v];
            l_run += psum;
          }
        }
      };
      const f32x16 sn = scores((const HSK_LDS char*)&s_tile[(T + 1) % kBufs32][0], side);
      pv((const HSK_LDS char*)&s_tile[T % kBufs32][0], pf);
      sc = sn;
    }
    softmax(sc, ntiles - 1, set_ref, pf);
    pv((const HSK_LDS char*)&s_tile[(ntiles - 1) % kBufs32][0], pf);
  };
  // the slow path's first pass: the true maximum over the partition's tiles
  auto max_pass = [&]() {
#pragma unroll
    for (int T = 0; T < kBufs32 - 1; ++T)
      if (T < ntiles) issue(T, T);
    for (int T = 0; T < ntiles; ++T) {
      wait_tile_barrier32(MY * min(ntiles - 1 - T, kBufs32 - 2));
      if (T + kBufs32 - 1 < ntiles) issue(T + kBufs32 - 1, (T + kBufs32 - 1) % kBufs32);
      f32x16 sc = scores((const HSK_LDS char*)&s_tile[T % kBufs32][0], no_side);
      const float tmax = tile_max(sc, T);
      m_ref = T == 0 ? tmax : fmaxf(m_ref, tmax);
    }
  };
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  if (ntiles > 0) full_pass(true, true);  // plan_attn makes no empty partition (and the combine skips a partition whose sum is 0)
  // every wave's loads are done (the last wait is for all of them) and every LDS read of the tiles is done;
  // any wave over the bound makes the workgroup redo the partition
  __syncthreads();
  if (__syncthreads_or(over)) {
    max_pass();
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
    l_run = 0.f;
    over = false;
    full_pass(false, false);
  }
  const float m_run = m_ref;

  // epilogue: lane holds head hbase + j, columns 32 cb + 8 (v / 4) + 4 h + v % 4.  The bf16 rows of the
  // wave's 32 heads are staged in the (now idle) tile buffers, 1,040 bytes apart so that the 32 heads of a
  // column step fall in different banks, then written out as whole 1,024-byte rows, 16 bytes per lane.
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const int head = hbase + j;
  const float inv = 1.f / l;
  const int64_t ps = ((int64_t)rq * a.split + sp) * a.H + head;
  constexpr int kRowStage = 1040;
  __syncthreads();  // every wave is done with the tile buffers
  HSK_LDS char* stage = (HSK_LDS char*)&s_tile[0][0] + wave * 32 * kRowStage;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 w;
      w.x = pack_bf16(oacc[cb][4 * g4] * inv, oacc[cb][4 * g4 + 1] * inv);
      w.y = pack_bf16(oacc[cb][4 * g4 + 2] * inv, oacc[cb][4 * g4 + 3] * inv);
      *(HSK_LDS u32x2*)(stage + j * kRowStage + (32 * cb + 8 * g4 + 4 * h) * 2) = w;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staged rows are written
  __builtin_amdgcn_wave_barrier();
  {
    // the wave's 32 output rows are contiguous: [head][512] bf16 from head hbase
    const int64_t row0 = a.split == 1 ? (int64_t)rq * a.H + hbase : ((int64_t)rq * a.split + sp) * a.H + hbase;
    char* dst = (char*)(a.split == 1 ? a.out : a.po) + row0 * kMlaDv * 2;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) {
      const u32x4 v = *(const HSK_LDS u32x4*)(stage + i * kRowStage + lane * 16);
      *(u32x4*)(dst + (int64_t)i * kMlaDv * 2 + lane * 16) = v;
    }
  }
  if (a.split > 1 && h == 0) {
    a.pm[ps] = m_run * kLn2;
    a.pl[ps] = l;
  }
}

// ------------------------------------------------------------------------------------------------------
// GQA pages (Quest-style page selection): 4 FLOP per byte, so this kernel is built for HBM bandwidth, not for
// the matrix cores.  Grid (split, request x KV head), 4 waves.  Tiles of 64 tokens (4 pages of 16) are
// gathered by page location into LDS with LDS-DMA loads, double-buffered; every wave takes one query head
// of the group:
//   scores:  lane t owns token t and takes the dot product of its key with the head's query held in
//            registers (v_dot2_f32_bf16 on bf16 pairs); the 16 key chunks of a token are XOR-swizzled by
//            the token so that 16 lanes reading chunk i hit 16 different bank groups;
//   softmax: online, fp32, exp2 domain, reference maximum moved only when exceeded by 2^8;
//   P.V:     lane l owns value dims 2l, 2l+1 and walks the 64 tokens in pairs: the pair's weights (bf16)
//            broadcast from one lane, the two tokens' values of a dim paired by a byte permute, v_dot2.
// ------------------------------------------------------------------------------------------------------
constexpr int kGqaTok = 64;                    // tokens per tile
constexpr int kGqaTokBytes = 512;              // one token: K 128 bf16 | V 128 bf16
constexpr int kGqaTileBytes = kGqaTok * kGqaTokBytes;  // 32 KB
constexpr int kGqaDma = kGqaTileBytes / 1024;  // 32 wave-wide loads per tile

struct GqaArgs {
  const uint16_t* q;
  const char* pool;
  const int32_t* locs;
  uint16_t* out;
  uint16_t* po;
  float* pm;
  float* pl;
  int32_t H, Hkv, k, page_tokens, row_bytes, split, pages_per_split;
  float scale_log2;
};

constexpr int kGqaMaxPages = 1024;             // pages of one partition (their locations are kept in LDS)

// maximum over the 64 lanes: within each row of 16 lanes by DPP row shifts (a lane without a source keeps
// its own value), then the four rows' last lanes by readlane
__device__ __forceinline__ float wave_max(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false))));
  const float a = fmaxf(__int_as_float(__builtin_amdgcn_readlane(v, 15)), __int_as_float(__builtin_amdgcn_readlane(v, 31)));
  const float b = fmaxf(__int_as_float(__builtin_amdgcn_readlane(v, 47)), __int_as_float(__builtin_amdgcn_readlane(v, 63)));
  return fmaxf(a, b);
}

__global__ __launch_bounds__(256) void gqa_attn_kernel(GqaArgs a) {
  __shared__ __attribute__((aligned(1024))) char s_tile[2][kGqaTileBytes];
  __shared__ int32_t s_loc[kGqaMaxPages];
  const int sp = blockIdx.x, unit = blockIdx.y;
  const int r = unit / a.Hkv, grp = unit % a.Hkv;
  const int hg = a.H / a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pt = a.page_tokens;
  const int p0 = sp * a.pages_per_split;
  const int npages = max(0, min(a.k, p0 + a.pages_per_split) - p0);
  const int ntok = npages * pt;
  const int ntiles = (ntok + kGqaTok - 1) / kGqaTok;
  const int32_t* locs = a.locs + (int64_t)unit * a.k + p0;
  const bool active = wave < hg;
  const int head = grp * hg + (active ? wave : 0);

  // query of this wave's head: 64 bf16 pairs, the same in every lane
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 qv[64];
  {
    const uint32_t* qh = (const uint32_t*)(a.q + ((int64_t)r * a.H + head) * 128);
#pragma unroll
    for (int i = 0; i < 64; ++i) qv[i] = __builtin_bit_cast(bf16x2, qh[i]);
  }
  // the partition's page locations go to LDS first: a tile's loads then wait for an LDS read, not for a
  // global one (whose in-order counter would also make them wait for the loads already in flight)
  // negative locations (a unit the resolve rejected) read page row 0: meaningless output, no load outside the pool
  for (int x = threadIdx.x; x < npages; x += 256) s_loc[x] = max(locs[x], 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const HSK_LDS char*)&s_tile[0][0];
  // DMA: wave-wide load j covers tile tokens 2j, 2j+1; lane l copies 16-byte slot l & 31 of token 2j + l / 32:
  // slots 0..15 are the key chunks, stored at position chunk ^ (token & 15), slots 16..31 the value chunks.
  // Pages of a power-of-two size up to a tile: a tile holds whole pages, so a lane's page within the tile and
  // its byte offset in the page row are the same for every tile; a load then costs one page index, one
  // location read and one 32 x 32 -> 64-bit multiply-add.  Other page sizes take the general form.
  constexpr int kGqaSlots = kGqaDma / 4;
  const bool whole_pages = (pt & (pt - 1)) == 0 && pt <= kGqaTok;
  const int ppt = whole_pages ? kGqaTok / pt : 0;  // pages per tile
  int pg_u[kGqaSlots];
  const char* base_u[kGqaSlots];
  if (whole_pages) {
#pragma unroll
    for (int u = 0; u < kGqaSlots; ++u) {
      const int t = 2 * (wave + 4 * u) + (lane >> 5);
      const int pos = lane & 31;
      const int chunk_off = pos < 16 ? ((pos ^ (t & 15)) << 4) : 256 + ((pos - 16) << 4);
      pg_u[u] = t / pt;
      base_u[u] = a.pool + (t % pt) * kGqaTokBytes + chunk_off;
    }
  }
  auto issue_pages = [&](int T, int b) {
#pragma unroll
    for (int u = 0; u < kGqaSlots; ++u) {
      int page = T * ppt + pg_u[u];
      page = page < npages ? page : 0;  // past the end: re-read page 0 (masked)
      const char* src = base_u[u] + (uint64_t)(uint32_t)s_loc[page] * (uint32_t)a.row_bytes;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + b * kGqaTileBytes + (wave + 4 * u) * 1024);
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
    }
  };
  auto issue_any = [&](int T, int b) {
#pragma unroll
    for (int u = 0; u < kGqaDma / 4; ++u) {
      const int j = wave + 4 * u;
      const int t = 2 * j + (lane >> 5);
      const int pos = lane & 31;
      int tok = T * kGqaTok + t;
      tok = tok < ntok ? tok : 0;  // past the end: re-read token 0 (masked)
      const int chunk_off = pos < 16 ? ((pos ^ (t & 15)) << 4) : 256 + ((pos - 16) << 4);
      const char* src = a.pool + (int64_t)s_loc[tok / pt] * a.row_bytes + (tok % pt) * kGqaTokBytes + chunk_off;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + b * kGqaTileBytes + j * 1024);  // wave-uniform
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
    }
  };

  auto issue = [&](int T, int b) {
    if (whole_pages) issue_pages(T, b); else issue_any(T, b);
  };

  float m_run = -INFINITY, l_lane = 0.f, o0 = 0.f, o1 = 0.f;
  if (ntiles > 0) issue(0, 0);
  for (int T = 0; T < ntiles; ++T) {
    const int b = T & 1;
    // tile T landed (this wave's loads, then every wave's) and every wave is done with tile T - 1, whose
    // buffer then takes tile T + 1 while tile T is computed
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (T + 1 < ntiles) issue(T + 1, b ^ 1);
    const HSK_LDS char* tile = (const HSK_LDS char*)&s_tile[b][0];
    if (active) {
      // scores: lane = token
      const HSK_LDS char* kt = tile + lane * kGqaTokBytes;
      const int x = lane & 15;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const HSK_LDS uint32_t* w = (const HSK_LDS uint32_t*)(kt + ((i ^ x) << 4));
        const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), qv[4 * i + 0], acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), qv[4 * i + 1], acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), qv[4 * i + 2], acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), qv[4 * i + 3], acc, false);
      }
      const float sc = T * kGqaTok + lane < ntok ? acc * a.scale_log2 : -INFINITY;
      const float tmax = wave_max(sc);
      if (tmax > m_run + 8.f) {  // wave-uniform: the reference maximum moves (always on the first tile)
        const float alpha = __builtin_amdgcn_exp2f(m_run - tmax);
        l_lane *= alpha;
        o0 *= alpha;
        o1 *= alpha;
        m_run = tmax;
      }
      const float p = __builtin_amdgcn_exp2f(sc - m_run);
      l_lane += p;
      // P.V: lane = value dims 2 lane, 2 lane + 1, tokens in pairs: lane t (t even) holds the weights of
      // tokens t and t + 1 as one bf16 pair, broadcast by one readlane; the two tokens' values of each dim
      // are paired with a byte permute and multiplied by v_dot2 (fp32 accumulation)
      const float pn = __shfl_down(p, 1, 64);
      const uint32_t pp = pack_bf16(p, pn);
      const HSK_LDS char* vt = tile + 256 + 4 * lane;
#pragma unroll
      for (int t = 0; t < kGqaTok; t += 2) {
        const bf16x2 w = __builtin_bit_cast(bf16x2, (uint32_t)__builtin_amdgcn_readlane((int)pp, t));
        const uint32_t v0 = *(const HSK_LDS uint32_t*)(vt + t * kGqaTokBytes);
        const uint32_t v1 = *(const HSK_LDS uint32_t*)(vt + (t + 1) * kGqaTokBytes);
        const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x05040100u);  // dim 2 lane of tokens t, t + 1
        const uint32_t hi = __builtin_amdgcn_perm(v1, v0, 0x07060302u);  // dim 2 lane + 1
        o0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lo), w, o0, false);
        o1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), w, o1, false);
      }
    }
  }
  if (!active) return;
  float l = l_lane;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  const float inv = 1.f / l;
  const uint32_t w = pack_bf16(o0 * inv, o1 * inv);
  if (a.split == 1) {
    *(uint32_t*)(a.out + ((int64_t)r * a.H + head) * 128 + 2 * lane) = w;
    return;
  }
  const int64_t ps = ((int64_t)r * a.split + sp) * a.H + head;
  *(uint32_t*)(a.po + ps * 128 + 2 * lane) = w;  // normalised by this partition's sum
  if (lane == 0) {
    a.pm[ps] = m_run * kLn2;  // natural-log units, as the combine expects
    a.pl[ps] = l;
  }
}

// ------------------------------------------------------------------------------------------------------
// combine: one wave per (query, head), 4 waves per block.  Partition s holds its output normalised by its
// own sum l_s, in bf16, with its maximum m_s: out = sum_s w_s o_s with w_s = l_s e^(m_s - M) / L and
// L = sum_s l_s e^(m_s - M).  Lane x owns the 16-byte chunk x (8 values) of the dv outputs (dv <= 512).
// Up to four partitions (the usual case) take one round trip: the rows, maxima and sums of all four are
// requested before any is used.  More partitions take a lane-parallel max and sum, then four rows at a time.
// With xcd set, block b serves query 8 ((b / 8) / (H / 4)) + b mod 8: blocks are dealt to the 8 XCDs by
// id mod 8, so a query's combine runs on the XCD whose MLA workgroups wrote its partials (same grouping as
// mla_block), and reads them from that XCD's L2 where they are still held.
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int dv, int xcd) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t RQ = (int64_t)a.R * a.Qmax;
  int64_t rq;
  int h;
  if (xcd) {
    const int hb = a.H >> 2;
    const int64_t j = blockIdx.x >> 3;
    rq = (j / hb) * 8 + (blockIdx.x & 7);
    h = 4 * (int)(j % hb) + wave;
    if (rq >= RQ) return;
  } else {
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= RQ * a.H) return;
    rq = item / a.H;
    h = (int)(item % a.H);
  }
  if (a.nq) {
    const int r = (int)(rq / a.Qmax), j = (int)(rq % a.Qmax);
    if (j >= a.nq[r]) return;
  }
  const int S = a.split;
  const int64_t p0 = rq * S * a.H + h;  // partition s of (rq, h) is p0 + s * H
  const bool mine = lane < (dv >> 3);
  if (S <= 4) {
    float mu[4], lu[4];
    u32x4 v[4];
    // the rows are loaded whatever the sums (every address is inside the partial buffers) and dropped after:
    // loaded only for a positive sum, each row load waited for its sum, two round trips instead of one
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t ps = p0 + (int64_t)(u < S ? u : 0) * a.H;
      mu[u] = u < S ? a.pm[ps] : -INFINITY;
      lu[u] = u < S ? a.pl[ps] : 0.f;
      v[u] = mine ? *(const u32x4*)(a.po + ps * dv + 8 * lane) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (!(u < S && lu[u] > 0.f)) v[u] = u32x4{0u, 0u, 0u, 0u};
    const float M = fmaxf(fmaxf(mu[0], mu[1]), fmaxf(mu[2], mu[3]));
    float w[4], L = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = (mu[u] == -INFINITY || !(lu[u] > 0.f)) ? 0.f : __expf(mu[u] - M) * lu[u];
      L += w[u];
    }
    const float invL = 1.f / L;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wu = w[u] * invL;
      const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(x[e] << 16) * wu;
        acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u) * wu;
      }
    }
    if (mine) {
      u32x4 o;
      o.x = pack_bf16(acc[0], acc[1]);
      o.y = pack_bf16(acc[2], acc[3]);
      o.z = pack_bf16(acc[4], acc[5]);
      o.w = pack_bf16(acc[6], acc[7]);
      *(u32x4*)(a.out + (rq * a.H + h) * dv + 8 * lane) = o;
    }
    return;
  }
  float M = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += 64)
    if (s0 + lane < S) M = fmaxf(M, a.pm[p0 + (int64_t)(s0 + lane) * a.H]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float L = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    if (s0 + lane < S) {
      const float m = a.pm[p0 + (int64_t)(s0 + lane) * a.H];
      const float lp = a.pl[p0 + (int64_t)(s0 + lane) * a.H];
      if (m != -INFINITY && lp > 0.f) L += __expf(m - M) * lp;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
  const float invL = 1.f / L;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 4) {
    float w[4];
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sidx = s0 + u;
      const int64_t ps = p0 + (int64_t)(sidx < S ? sidx : 0) * a.H;
      const float m = sidx < S ? a.pm[ps] : -INFINITY;
      const float lp = sidx < S ? a.pl[ps] : 0.f;
      w[u] = (m == -INFINITY || !(lp > 0.f)) ? 0.f : __expf(m - M) * lp * invL;
      v[u] = mine ? *(const u32x4*)(a.po + ps * dv + 8 * lane) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (w[u] == 0.f) v[u] = u32x4{0u, 0u, 0u, 0u};   // loaded whatever the weight, dropped here
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(x[e] << 16) * w[u];
        acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u) * w[u];
      }
    }
  }
  if (mine) {
    u32x4 o;
    o.x = pack_bf16(acc[0], acc[1]);
    o.y = pack_bf16(acc[2], acc[3]);
    o.z = pack_bf16(acc[4], acc[5]);
    o.w = pack_bf16(acc[6], acc[7]);
    *(u32x4*)(a.out + (rq * a.H + h) * dv + 8 * lane) = o;
  }
}

// Grid of combine_kernel: blocks of four (query, head) waves, XCD-grouped when the heads come in fours.
static void launch_combine(const AttnArgs& a, int64_t RQ, hipStream_t s) {
  const int xcd = (a.H % 4 == 0 && RQ >= 8) ? 1 : 0;
  const int64_t blocks = xcd ? 8 * (int64_t)(a.H / 4) * ((RQ + 7) / 8) : (RQ * a.H + 3) / 4;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, a.dv, xcd);
}

// Launch plan of one attention call: split-k partitions and, for MLA, the wave-pair shape.
struct AttnPlan {
  int split, rows_per_split;
  int nhb, npair, hgroups;  // MLA: 16-head blocks per wave pair, pairs per workgroup, head groups
  int nw32;                 // MLA with heads % 64 == 0: waves (32 heads each) of mla32_kernel, same head groups
  int64_t po_bytes, pm_bytes, scratch;
};

// max_rows bounds the rows of one partition (the fused kernel keeps two location arrays in LDS).
static bool plan_attn(const hsk_attn_desc* d, AttnPlan* p, int max_rows = kMaxSplitRows) {
  if (!d || d->num_requests < 1 || d->max_queries < 1 || d->heads < 1 || d->top_k < 1 || d->split < 0) return false;
  // the kernels take the maximum of the raw scores and scale it afterwards, which is the maximum of the
  // scaled scores only for a positive scale
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return false;
  const int64_t RQ = (int64_t)d->num_requests * d->max_queries;
  const int k = d->top_k;
  if (d->kind == HSK_ATTN_MLA) {
    if (d->kv_heads != 1 || d->dk != kMlaDk || d->dv != kMlaDv || d->row_elems < kMlaDk || d->row_elems % 8 ||
        d->heads % 16 || d->page_tokens != 1)
      return false;
    p->nhb = d->heads % 32 == 0 ? 2 : 1;
    const int units = d->heads / (16 * p->nhb);
    p->npair = units % 4 == 0 ? 4 : units % 2 == 0 ? 2 : 1;
    p->hgroups = units / p->npair;
    // 32 heads per wave: 4 waves when the heads come in 128s, else 2 (64s); the head groups are the same
    p->nw32 = d->heads % 128 == 0 ? 4 : d->heads % 64 == 0 ? 2 : 0;
    const int min_split = (k + max_rows - 1) / max_rows;
    if (d->split > 0) {
      // a forced split is an upper bound: rows_per_split = ceil(k / split), and the partitions are the
      // ceil(k / rows_per_split) non-empty runs of that many rows (k = 2,048 with split = 100 gives 98)
      p->rows_per_split = (k + d->split - 1) / d->split;
      if (p->rows_per_split > max_rows) return false;
      p->split = (k + p->rows_per_split - 1) / p->rows_per_split;
    } else {
      // about one workgroup per compute unit (a workgroup fills a CU's LDS), tiles of whole 32-row blocks
      const int64_t base = RQ * p->hgroups;
      int64_t s = (256 + base - 1) / base;
      const int64_t max_s = (k + kTile - 1) / kTile;
      s = s > max_s ? max_s : s;
      s = s < min_split ? min_split : s;
      int rps = (int)((k + s - 1) / s);
      if (s > 1) rps = (rps + kTile - 1) / kTile * kTile;
      if (rps > max_rows) rps = max_rows;
      p->rows_per_split = rps;
      p->split = (k + rps - 1) / rps;
    }
    // one-dimensional grid: its work-items must stay below 2^31
    if ((int64_t)p->split * p->hgroups * (RQ + 8) * 128 * p->npair >= (int64_t(1) << 31)) return false;
  } else if (d->kind == HSK_ATTN_GQA) {
    if (d->max_queries != 1 || d->kv_heads < 1 || d->heads % d->kv_heads || d->heads / d->kv_heads > 4 ||
        d->dk != 128 || d->dv != 128 || d->page_tokens < 1 || d->row_elems != d->page_tokens * 2 * d->dk)
      return false;
    p->nhb = p->npair = p->hgroups = 0;
    if (d->split > 0) {
      p->split = d->split;
    } else {
      // about four workgroups per CU at a time (a workgroup holds 68 KB of LDS: two fit)
      const int64_t base = (int64_t)d->num_requests * d->kv_heads;
      int64_t s = (1024 + base - 1) / base;
      s = s < 1 ? 1 : s;
      s = s < (k + kGqaMaxPages - 1) / kGqaMaxPages ? (k + kGqaMaxPages - 1) / kGqaMaxPages : s;
      p->split = (int)(s > k ? k : s);
    }
    // every partition holds at least one page: with rows_per_split = ceil(k / split) pages each, only
    // ceil(k / rows_per_split) partitions are non-empty (R = 3, Hkv = 8, k = 100 asks for 43 and gets 34)
    p->rows_per_split = (k + p->split - 1) / p->split;
    if (p->rows_per_split > kGqaMaxPages) return false;
    p->split = (k + p->rows_per_split - 1) / p->rows_per_split;
  } else {
    return false;
  }
  const int64_t parts = RQ * p->split * d->heads;
  const bool partials = p->split > 1;
  p->po_bytes = partials ? (parts * d->dv * 2 + 255) / 256 * 256 : 0;
  p->pm_bytes = partials ? (parts * 4 + 255) / 256 * 256 : 0;
  p->scratch = p->po_bytes + 2 * p->pm_bytes;
  if (p->scratch < 256) p->scratch = 256;
  return true;
}

template <int NW>
static void launch_mla32(MlaArgs m, const AttnPlan& p, int64_t RQ, hipStream_t s) {
  const int64_t G = (int64_t)p.split * p.hgroups;
  m.hgroups = p.hgroups;
  m.RQ = (int32_t)RQ;
  m.xcd_groups = (G > 1 && RQ >= 8) ? (int32_t)G : 0;
  const int64_t blocks = m.xcd_groups ? 8 * G * ((RQ + 7) / 8) : G * RQ;
  hipLaunchKernelGGL((mla32_kernel<NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, m);
}

// Fills the launch fields of m (head groups, queries, XCD grouping) and launches the MLA kernel.
template <int NHB, int NPAIR, bool FUSED = false>
static void launch_mla(MlaArgs m, const AttnPlan& p, int64_t RQ, hipStream_t s) {
  const int64_t G = (int64_t)p.split * p.hgroups;
  m.hgroups = p.hgroups;
  m.RQ = (int32_t)RQ;
  m.xcd_groups = (G > 1 && RQ >= 8) ? (int32_t)G : 0;
  const int64_t blocks = m.xcd_groups ? 8 * G * ((RQ + 7) / 8) : G * RQ;
  hipLaunchKernelGGL((mla_mfma_kernel<NHB, NPAIR, FUSED>), dim3((unsigned)blocks), dim3(128 * NPAIR), 0, s, m);
}

static hsk_status launch_attn(const hsk_attn_desc* d, const AttnPlan& p, const void* d_q, const void* d_pool,
                              const int32_t* d_locs, const int32_t* d_nq, void* d_out, void* d_scratch,
                              hipStream_t s);

// Split-k scratch of hsk_sparse_decode_attn_noalloc, for callers that cannot allocate.  In host code the
// name `scratch` is only a host-side handle of the array: kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device with that device current and kept in
// g_scratch_dev (each GPU holds its own copy of the array, at its own address).
constexpr size_t kNoAllocScratchBytes = HSK_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];

static hsk_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HSK_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return HSK_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return HSK_EHIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return HSK_OK;
}

}  // namespace hsk

using namespace hsk;

extern "C" {

hsk_status hsk_attn_scratch_bytes(const hsk_attn_desc* d, size_t* bytes) {
  AttnPlan p, pf;
  if (!bytes || !plan_attn(d, &p)) return HSK_EINVAL;
  *bytes = (size_t)p.scratch;
  // enough for the fused resolve + attend as well, whose partitions hold at most kMaxFusedRows rows
  if (d->kind == HSK_ATTN_MLA && d->max_queries == 1 && plan_attn(d, &pf, kMaxFusedRows) && pf.scratch > p.scratch)
    *bytes = (size_t)pf.scratch;
  return HSK_OK;
}

hsk_status hsk_sparse_decode_attn(const hsk_attn_desc* d, const void* d_q, const void* d_pool, const int32_t* d_locs,
                                  const int32_t* d_nq, void* d_out, void* d_scratch, size_t scratch_bytes,
                                  hsk_stream_t stream) {
  AttnPlan p;
  if (!plan_attn(d, &p) || !d_q || !d_pool || !d_locs || !d_out || !d_scratch) return HSK_EINVAL;
  if (scratch_bytes < (size_t)p.scratch || ((uintptr_t)d_scratch % 256)) return HSK_EINVAL;
  return launch_attn(d, p, d_q, d_pool, d_locs, d_nq, d_out, d_scratch, (hipStream_t)stream);
}

hsk_status hsk_sparse_decode_attn_noalloc(const hsk_attn_desc* d, const void* d_q, const void* d_pool,
                                          const int32_t* d_locs, const int32_t* d_nq, void* d_out,
                                          hsk_stream_t stream) {
  AttnPlan p;
  if (!plan_attn(d, &p) || !d_q || !d_pool || !d_locs || !d_out) return HSK_EINVAL;
  if ((uint64_t)p.scratch > (uint64_t)kNoAllocScratchBytes) return HSK_ESCRATCH;
  void* buf = nullptr;
  const hsk_status st = noalloc_scratch(&buf);
  if (st != HSK_OK) return st;
  return launch_attn(d, p, d_q, d_pool, d_locs, d_nq, d_out, buf, (hipStream_t)stream);
}

}  // extern "C"

namespace hsk {

// One attention call on stream s: the MLA or GQA kernel, then the split-k combine when there are several
// partitions.  The plan p and the scratch (>= p.scratch bytes, 256-byte aligned) are checked by the caller.
static hsk_status launch_attn(const hsk_attn_desc* d, const AttnPlan& p, const void* d_q, const void* d_pool,
                              const int32_t* d_locs, const int32_t* d_nq, void* d_out, void* d_scratch,
                              hipStream_t s) {
  const int64_t RQ = (int64_t)d->num_requests * d->max_queries;
  AttnArgs a;
  a.q = (const uint16_t*)d_q;
  a.pool = (const char*)d_pool;
  a.locs = d_locs;
  a.nq = d->kind == HSK_ATTN_MLA ? d_nq : nullptr;
  a.out = (uint16_t*)d_out;
  a.R = d->num_requests; a.Qmax = d->max_queries; a.H = d->heads; a.Hkv = d->kv_heads;
  a.dk = d->dk; a.dv = d->dv; a.k = d->top_k; a.row_elems = d->row_elems; a.page_tokens = d->page_tokens;
  a.split = p.split;
  a.rows_per_split = p.rows_per_split;
  a.scale = d->scale;
  a.po = (uint16_t*)d_scratch;
  a.pm = (float*)((char*)d_scratch + p.po_bytes);
  a.pl = (float*)((char*)d_scratch + p.po_bytes + p.pm_bytes);
  if (d->kind == HSK_ATTN_MLA) {
    MlaArgs m;
    m.q = a.q; m.pool = a.pool; m.locs = a.locs; m.nq = a.nq; m.out = a.out;
    m.po = a.po; m.pm = a.pm; m.pl = a.pl;
    m.Qmax = d->max_queries; m.H = d->heads; m.k = d->top_k; m.row_bytes = d->row_elems * 2;
    m.split = p.split; m.rows_per_split = p.rows_per_split;
    m.scale_log2 = d->scale * kLog2e;
    m.fill = nullptr; m.host = nullptr; m.host_req_stride = 0;
    if (p.nw32 == 4) launch_mla32<4>(m, p, RQ, s);
    else if (p.nw32 == 2) launch_mla32<2>(m, p, RQ, s);
    else if (p.nhb == 2 && p.npair == 4) launch_mla<2, 4>(m, p, RQ, s);
    else if (p.nhb == 2 && p.npair == 2) launch_mla<2, 2>(m, p, RQ, s);
    else if (p.nhb == 2) launch_mla<2, 1>(m, p, RQ, s);
    else launch_mla<1, 1>(m, p, RQ, s);
    HSK_HIP(hipGetLastError());
    if (p.split == 1) return HSK_OK;
  } else {
    GqaArgs gq;
    gq.q = a.q; gq.pool = a.pool; gq.locs = a.locs; gq.out = a.out; gq.po = a.po; gq.pm = a.pm; gq.pl = a.pl;
    gq.H = d->heads; gq.Hkv = d->kv_heads; gq.k = d->top_k; gq.page_tokens = d->page_tokens;
    gq.row_bytes = d->row_elems * 2; gq.split = p.split; gq.pages_per_split = p.rows_per_split;
    gq.scale_log2 = d->scale * kLog2e;
    hipLaunchKernelGGL(gqa_attn_kernel, dim3(p.split, (int64_t)d->num_requests * d->kv_heads), dim3(256), 0, s, gq);
    HSK_HIP(hipGetLastError());
    if (p.split == 1) return HSK_OK;
  }
  launch_combine(a, RQ, s);
  HSK_HIP(hipGetLastError());
  return HSK_OK;
}

hsk_status check_mla_fused(const hsk_attn_desc* d, const void* scratch, size_t scratch_bytes) {
  AttnPlan p;
  if (!d || !scratch || !plan_attn(d, &p, kMaxFusedRows) || d->kind != HSK_ATTN_MLA || d->max_queries != 1)
    return HSK_EINVAL;
  if (scratch_bytes < (size_t)p.scratch || ((uintptr_t)scratch % 256)) return HSK_EINVAL;
  return HSK_OK;
}

hsk_status launch_mla_fused(const hsk_attn_desc* d, const void* q, const char* pool, const int32_t* locs,
                            const int32_t* fill, const char* host, int64_t host_req_stride, void* out,
                            void* scratch, size_t scratch_bytes, hipStream_t s) {
  AttnPlan p;
  if (check_mla_fused(d, scratch, scratch_bytes) != HSK_OK || !q || !pool || !locs || !fill || !host || !out)
    return HSK_EINVAL;
  plan_attn(d, &p, kMaxFusedRows);
  const int64_t RQ = d->num_requests;
  MlaArgs m;
  m.q = (const uint16_t*)q; m.pool = pool; m.locs = locs; m.nq = nullptr; m.out = (uint16_t*)out;
  m.po = (uint16_t*)scratch;
  m.pm = (float*)((char*)scratch + p.po_bytes);
  m.pl = (float*)((char*)scratch + p.po_bytes + p.pm_bytes);
  m.fill = fill; m.host = host; m.host_req_stride = host_req_stride;
  m.Qmax = 1; m.H = d->heads; m.k = d->top_k; m.row_bytes = d->row_elems * 2;
  m.split = p.split; m.rows_per_split = p.rows_per_split;
  m.scale_log2 = d->scale * kLog2e;
  if (p.nhb == 2 && p.npair == 4) launch_mla<2, 4, true>(m, p, RQ, s);
  else if (p.nhb == 2 && p.npair == 2) launch_mla<2, 2, true>(m, p, RQ, s);
  else if (p.nhb == 2) launch_mla<2, 1, true>(m, p, RQ, s);
  else launch_mla<1, 1, true>(m, p, RQ, s);
  HSK_HIP(hipGetLastError());
  if (p.split == 1) return HSK_OK;
  AttnArgs a;
  a.q = m.q; a.pool = pool; a.locs = locs; a.nq = nullptr; a.out = m.out;
  a.R = d->num_requests; a.Qmax = 1; a.H = d->heads; a.Hkv = 1;
  a.dk = d->dk; a.dv = d->dv; a.k = d->top_k; a.row_elems = d->row_elems; a.page_tokens = 1;
  a.split = p.split; a.rows_per_split = p.rows_per_split; a.scale = d->scale;
  a.po = m.po; a.pm = m.pm; a.pl = m.pl;
  launch_combine(a, RQ, s);
  HSK_HIP(hipGetLastError());
  return HSK_OK;
}

}  // namespace hsk
