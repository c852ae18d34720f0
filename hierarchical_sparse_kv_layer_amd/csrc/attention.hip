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

#include "hsk_internal.h"

namespace hsk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct AttnArgs {
  const uint16_t* q;
  const char* pool;
  const int32_t* locs;
  const int32_t* nq;
  uint16_t* out;
  float* po;   // [RQ][split][H][dv]
  float* pm;   // [RQ][split][H]
  float* pl;   // [RQ][split][H]
  int32_t R, Qmax, H, Hkv, dk, dv, k, row_elems, page_tokens, split, rows_per_split;
  float scale;
};

// ------------------------------------------------------------------------------------------------------
// MLA: grid (split, H / kMlaHeads, R * Qmax), 256 threads.  A block holds kMlaHeads query heads in LDS
// (fp32) and streams its partition of rows through LDS in tiles of kMlaTile rows.
// ------------------------------------------------------------------------------------------------------
constexpr int kMlaThreads = 256;
constexpr int kMlaHeads = 16;
constexpr int kMlaTile = 32;
constexpr int kMlaMaxDk = 576;
constexpr int kMlaMaxDv = 512;
constexpr int kMlaRowWords = kMlaMaxDk / 2 + 2;  // bf16 pairs per LDS row, +2 words against bank conflicts

__global__ __launch_bounds__(kMlaThreads) void mla_attn_kernel(AttnArgs a) {
  __shared__ float s_q[kMlaHeads][kMlaMaxDk];
  __shared__ uint32_t s_row[kMlaTile][kMlaRowWords];
  __shared__ float s_p[kMlaHeads][kMlaTile];

  const int sp = blockIdx.x, hg = blockIdx.y, rq = blockIdx.z;
  const int r = rq / a.Qmax, j = rq % a.Qmax;
  if (a.nq && j >= a.nq[r]) return;
  const int tid = threadIdx.x;
  const int i0 = sp * a.rows_per_split;
  const int i1 = min(a.k, i0 + a.rows_per_split);
  const int h0 = hg * kMlaHeads;
  const int dk = a.dk, dv = a.dv;

  const uint16_t* q = a.q + ((int64_t)rq * a.H + h0) * dk;
  for (int x = tid; x < kMlaHeads * dk; x += kMlaThreads) s_q[x / dk][x % dk] = bf16f(q[x]);

  // output ownership: head hh = tid / 16, columns c * 16 + sub (interleaved -> conflict-free LDS reads)
  const int hh = tid >> 4, sub = tid & 15;
  const int ncol = (dv + 15) >> 4;  // <= 32
  float o[kMlaMaxDv / 16];
#pragma unroll
  for (int c = 0; c < kMlaMaxDv / 16; ++c) o[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t* locs = a.locs + (int64_t)rq * a.k;
  const int row_bytes = a.row_elems * 2;
  const int chunks8 = dk / 4;  // 8-byte chunks of the key part

  for (int t0 = i0; t0 < i1; t0 += kMlaTile) {
    const int nt = min(kMlaTile, i1 - t0);
    __syncthreads();
    for (int x = tid; x < nt * chunks8; x += kMlaThreads) {
      const int i = x / chunks8, c = x % chunks8;
      const u32x2* src = (const u32x2*)(a.pool + (int64_t)locs[t0 + i] * row_bytes) + c;
      const u32x2 w = *src;
      s_row[i][2 * c] = w.x;
      s_row[i][2 * c + 1] = w.y;
    }
    __syncthreads();
    // scores: kMlaHeads x nt dot products of length dk
    for (int x = tid; x < kMlaHeads * kMlaTile; x += kMlaThreads) {
      const int h = x / kMlaTile, i = x % kMlaTile;
      float acc = -INFINITY;
      if (i < nt) {
        acc = 0.f;
        const float* qh = s_q[h];
        const uint32_t* row = s_row[i];
        for (int d2 = 0; d2 < dk / 2; ++d2) {
          const uint32_t w = row[d2];
          acc = fmaf(qh[2 * d2], bf16lo(w), acc);
          acc = fmaf(qh[2 * d2 + 1], bf16hi(w), acc);
        }
        acc *= a.scale;
      }
      s_p[h][i] = acc;
    }
    __syncthreads();
    // online softmax and P.V for head hh over this tile
    float tmax = -INFINITY;
    for (int i = 0; i < nt; ++i) tmax = fmaxf(tmax, s_p[hh][i]);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < kMlaMaxDv / 16; ++c) o[c] *= alpha;
    for (int i = 0; i < nt; ++i) {
      const float p = __expf(s_p[hh][i] - m_new);
      l_run += p;
      const uint16_t* v = (const uint16_t*)s_row[i];
#pragma unroll
      for (int c = 0; c < kMlaMaxDv / 16; ++c) {
        const int col = c * 16 + sub;
        if (c < ncol && col < dv) o[c] = fmaf(p, bf16f(v[col]), o[c]);
      }
    }
    m_run = m_new;
  }
  // partial results
  const int64_t ps = ((int64_t)rq * a.split + sp) * a.H + h0 + hh;
  float* po = a.po + ps * dv;
#pragma unroll
  for (int c = 0; c < kMlaMaxDv / 16; ++c) {
    const int col = c * 16 + sub;
    if (c < ncol && col < dv) po[col] = o[c];
  }
  if (sub == 0) {
    a.pm[ps] = m_run;
    a.pl[ps] = l_run;
  }
}

// ------------------------------------------------------------------------------------------------------
// GQA pages: grid (split, R * Hkv), 64 x (H / Hkv) threads: one wave per query head, each lane owns two of
// the 128 head dims; scores are wave reductions, values accumulate per lane.
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gqa_attn_kernel(AttnArgs a) {
  const int sp = blockIdx.x, unit = blockIdx.y;
  const int r = unit / a.Hkv, g = unit % a.Hkv;
  const int gsize = a.H / a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = g * gsize + wave;
  const int dh = a.dk;            // 128: two dims per lane
  const int i0 = sp * a.rows_per_split;
  const int i1 = min(a.k, i0 + a.rows_per_split);
  const uint16_t* qh = a.q + ((int64_t)r * a.H + h) * dh;
  const uint32_t qw = *(const uint32_t*)(qh + 2 * lane);
  const float q0 = bf16lo(qw), q1 = bf16hi(qw);
  const int32_t* locs = a.locs + (int64_t)unit * a.k;
  const int row_bytes = a.row_elems * 2;
  const int tok_bytes = 4 * dh;
  float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
  for (int i = i0; i < i1; ++i) {
    const char* page = a.pool + (int64_t)locs[i] * row_bytes;
    for (int t = 0; t < a.page_tokens; ++t) {
      const char* tok = page + (int64_t)t * tok_bytes;
      const uint32_t kw = *(const uint32_t*)(tok + 4 * lane);
      const uint32_t vw = *(const uint32_t*)(tok + 2 * dh + 4 * lane);
      float s = q0 * bf16lo(kw) + q1 * bf16hi(kw);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      s *= a.scale;
      const float m_new = fmaxf(m_run, s);
      const float alpha = __expf(m_run - m_new);
      const float p = __expf(s - m_new);
      l_run = l_run * alpha + p;
      o0 = o0 * alpha + p * bf16lo(vw);
      o1 = o1 * alpha + p * bf16hi(vw);
      m_run = m_new;
    }
  }
  const int64_t ps = ((int64_t)r * a.split + sp) * a.H + h;  // GQA: RQ index = request
  a.po[ps * dh + 2 * lane] = o0;
  a.po[ps * dh + 2 * lane + 1] = o1;
  if (lane == 0) {
    a.pm[ps] = m_run;
    a.pl[ps] = l_run;
  }
}

// ------------------------------------------------------------------------------------------------------
// combine: grid (RQ, H), 128 threads
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a, int dv) {
  const int rq = blockIdx.x, h = blockIdx.y;
  if (a.nq) {
    const int r = rq / a.Qmax, j = rq % a.Qmax;
    if (j >= a.nq[r]) return;
  }
  float M = -INFINITY;
  for (int s = 0; s < a.split; ++s) M = fmaxf(M, a.pm[((int64_t)rq * a.split + s) * a.H + h]);
  float L = 0.f;
  for (int s = 0; s < a.split; ++s) {
    const int64_t ps = ((int64_t)rq * a.split + s) * a.H + h;
    const float m = a.pm[ps];
    L += (m == -INFINITY) ? 0.f : __expf(m - M) * a.pl[ps];
  }
  const float invL = 1.f / L;
  for (int c = threadIdx.x; c < dv; c += 128) {
    float acc = 0.f;
    for (int s = 0; s < a.split; ++s) {
      const int64_t ps = ((int64_t)rq * a.split + s) * a.H + h;
      const float m = a.pm[ps];
      if (m != -INFINITY) acc += __expf(m - M) * a.po[ps * dv + c];
    }
    a.out[((int64_t)rq * a.H + h) * dv + c] = f2bf16(acc * invL);
  }
}

static int auto_split(const hsk_attn_desc* d) {
  if (d->split > 0) return d->split;
  if (d->kind == HSK_ATTN_MLA) {
    // enough workgroups for 256 CUs: (R * Qmax) * (H / 16) * split >= ~2048
    const int64_t base = (int64_t)d->num_requests * d->max_queries * (d->heads / kMlaHeads);
    int s = (int)((2048 + base - 1) / base);
    s = s < 1 ? 1 : s;
    const int max_s = (d->top_k + kMlaTile - 1) / kMlaTile;
    return s > max_s ? max_s : s;
  }
  const int64_t base = (int64_t)d->num_requests * d->kv_heads;
  int s = (int)((2048 + base - 1) / base);
  s = s < 1 ? 1 : s;
  return s > d->top_k ? d->top_k : s;
}

static bool valid_attn(const hsk_attn_desc* d) {
  if (!d || d->num_requests < 1 || d->max_queries < 1 || d->heads < 1 || d->top_k < 1 || d->split < 0) return false;
  if (d->kind == HSK_ATTN_MLA) {
    if (d->kv_heads != 1 || d->dk < 2 || d->dk > kMlaMaxDk || d->dk % 4 || d->dv < 1 || d->dv > d->dk ||
        d->dv > kMlaMaxDv || d->row_elems < d->dk || d->row_elems % 8 || d->heads % kMlaHeads || d->page_tokens != 1)
      return false;
    return true;
  }
  if (d->kind == HSK_ATTN_GQA) {
    if (d->max_queries != 1 || d->kv_heads < 1 || d->heads % d->kv_heads || d->heads / d->kv_heads > 4 ||
        d->dk != 128 || d->dv != 128 || d->page_tokens < 1 || d->row_elems != d->page_tokens * 2 * d->dk)
      return false;
    return true;
  }
  return false;
}

}  // namespace hsk

using namespace hsk;

extern "C" {

hsk_status hsk_attn_scratch_bytes(const hsk_attn_desc* d, size_t* bytes) {
  if (!valid_attn(d) || !bytes) return HSK_EINVAL;
  const int64_t split = auto_split(d);
  const int64_t RQ = (int64_t)d->num_requests * d->max_queries;
  const int64_t parts = RQ * split * d->heads;
  const int64_t po = (parts * d->dv * 4 + 255) / 256 * 256;
  const int64_t pm = (parts * 4 + 255) / 256 * 256;
  *bytes = (size_t)(po + 2 * pm);
  return HSK_OK;
}

hsk_status hsk_sparse_decode_attn(const hsk_attn_desc* d, const void* d_q, const void* d_pool, const int32_t* d_locs,
                                  const int32_t* d_nq, void* d_out, void* d_scratch, size_t scratch_bytes,
                                  hsk_stream_t stream) {
  if (!valid_attn(d) || !d_q || !d_pool || !d_locs || !d_out || !d_scratch) return HSK_EINVAL;
  size_t need = 0;
  hsk_attn_scratch_bytes(d, &need);
  if (scratch_bytes < need || ((uintptr_t)d_scratch % 256)) return HSK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  AttnArgs a;
  a.q = (const uint16_t*)d_q;
  a.pool = (const char*)d_pool;
  a.locs = d_locs;
  a.nq = d->kind == HSK_ATTN_MLA ? d_nq : nullptr;
  a.out = (uint16_t*)d_out;
  a.R = d->num_requests; a.Qmax = d->max_queries; a.H = d->heads; a.Hkv = d->kv_heads;
  a.dk = d->dk; a.dv = d->dv; a.k = d->top_k; a.row_elems = d->row_elems; a.page_tokens = d->page_tokens;
  a.split = auto_split(d);
  a.rows_per_split = (d->top_k + a.split - 1) / a.split;
  a.scale = d->scale;
  const int64_t RQ = (int64_t)d->num_requests * d->max_queries;
  const int64_t parts = RQ * a.split * d->heads;
  const int64_t po_bytes = (parts * d->dv * 4 + 255) / 256 * 256;
  const int64_t pm_bytes = (parts * 4 + 255) / 256 * 256;
  a.po = (float*)d_scratch;
  a.pm = (float*)((char*)d_scratch + po_bytes);
  a.pl = (float*)((char*)d_scratch + po_bytes + pm_bytes);
  if (d->kind == HSK_ATTN_MLA) {
    hipLaunchKernelGGL(mla_attn_kernel, dim3(a.split, d->heads / kMlaHeads, RQ), dim3(kMlaThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(gqa_attn_kernel, dim3(a.split, (int64_t)d->num_requests * d->kv_heads),
                       dim3(64 * (d->heads / d->kv_heads)), 0, s, a);
  }
  HSK_HIP(hipGetLastError());
  hipLaunchKernelGGL(combine_kernel, dim3(RQ, d->heads), dim3(128), 0, s, a, d->dv);
  HSK_HIP(hipGetLastError());
  return HSK_OK;
}

}  // extern "C"
