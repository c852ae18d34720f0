// Resolve and row-movement kernels for gfx950.
//
// resolve_kernel: one 1024-thread workgroup per request.  It implements the fused resolve of "HiSparse:
// Scaling Sparse-Attention Decoding with Hierarchical KV Cache Management" (section 3.4: stage the
// selection, mark hot slots hit or evictable, scan marks to pick victims and update LRU metadata, publish
// locations) with the residency-aware order of "Adaptive DHiSparse: Speculative Decoding over a
// Load-Adaptive KV Hierarchy" (section 3.2 / Figure 2: tail and ready optional pages first) and the
// multi-query union of its section 3.3 (Eqs. 5-6: each distinct missing row once, overflow to staging).
//
// How the phases map to CDNA4:
//   * the selection is probed through the page table (one load per selected row) instead of hashing the
//     selection and probing every slot: hits set bits in a B-bit LDS bitmap with LDS atomics;
//   * duplicate misses are collapsed without a hash: each missing selection f does atomicMin(pt[p],
//     INT_MIN + f), so the page-table word itself ends holding the first occurrence (order-independent,
//     hence deterministic); the first-occurrence flags are then compacted with wave ballots and a
//     block-wide prefix sum, in ascending f, giving every distinct miss its index in miss order;
//   * victims come from the per-request slot order kept in (rec, slot) order: a ballot/prefix scan over
//     that list, skipping hit slots, yields the oldest unselected slots in order -- no sort, no atomics;
//   * the new order is written as [unselected non-victims in old order][fills by slot][hits by slot],
//     which is exactly the ascending (rec, slot) order once fills get 2e and hits 2e+1 (epochs increase).
// The host-to-device copies of the missing rows run at the end of the same kernel (each workgroup copies its
// request's rows); gather_kernel, which spreads a plan's rows evenly over all its waves, replays a recorded
// plan into another source's pool.
#include <climits>

#include <hip/hip_ext.h>

#include "hsk_internal.h"

namespace hsk {

// Everything a resolve workgroup shares through global memory (its request's page table, locations and
// miss plan) is touched by that workgroup alone during the kernel, so workgroup scope is enough: on this
// multi-XCD part an agent-scope fence would write back and invalidate the whole L2.  A value that another
// thread changed with an atomic is read back with an atomic (it executes at L2), never a plain load that
// could hit a line this CU cached before the atomic.
// LDS writes of this wave complete, then a workgroup barrier; global stores stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int32_t rmw_read(int32_t* p) {
  return __hip_atomic_fetch_or(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void claim_min(int32_t* p, int32_t v) {
  __hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within each row of 16 lanes by DPP row
// shifts (lanes without a source add 0), then each row adds the totals of the rows before it, read with
// readlane from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Exclusive prefix sum of small non-negative ints over the workgroup in thread order (LDS-only barriers:
// global stores of the caller stay in flight).  Must be called by every thread of the block.  The wave
// totals go to s_wsum, which has no barrier after its reads: two scans in a row use different buffers (a
// scan's first barrier is passed only once every thread has read the buffer of the scan before).
__device__ __forceinline__ int block_sum_scan(int v, int* total, int* s_wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_wsum[wave] = x;
  lds_barrier();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kResolveWaves; ++w) {
    const int c = s_wsum[w];
    base += (w < wave) ? c : 0;
    tot += c;
  }
  *total = tot;
  return base + x - v;
}

enum { kDirectNone = 0, kDirectTail = 1, kDirectOpt = 2 };

// Direct pass of one selection (Adaptive DHiSparse section 3.2, callout 1): tail, then a ready complete
// optional page; returns the class and sets *loc for direct rows.
__device__ __forceinline__ int classify(const ResolveArgs& a, int r, int64_t n, const int32_t* opt, int32_t p,
                                        int32_t* loc) {
  if (p >= n - a.T) {
    *loc = (int32_t)((int64_t)a.R * a.B + (int64_t)r * a.T + (p % a.T));
    return kDirectTail;
  }
  if (opt != nullptr && (int64_t)(p / a.P) < n / a.P) {
    const int32_t g = opt[p / a.P];
    if (g >= 0) {
      *loc = (int32_t)(a.opt_base + (int64_t)g * a.P + (p % a.P));
      return kDirectOpt;
    }
  }
  return kDirectNone;
}

// Fused resolve + attend: when a.fill is set, fill[f] tells the attention kernel where selection f's row
// comes from in this call: -1 if it is resident (pool row locs[f]), else 2 p + first for a row copied from
// host position p in this call, first = 1 on the first occurrence (the one that writes it into locs[f]);
// positions stay below 2^30 on this path.
// Per-selection codes while a call runs (kept in registers when the request has at most kPer * threads
// selections, else in the location array, which then doubles as scratch):
//   >= 0              final location (a direct row or a hot hit)
//   kCodeMiss         a missing position, before its claim is read back
//   INT_MIN + f0      a repeated miss whose first occurrence is selection f0
//   -2 - i            the first occurrence of distinct miss i (also stored at locs[f0] for repeats to read)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int32_t kCodeMiss = -1;
constexpr int kPer = 4;                                   // contiguous selections per thread per round
constexpr int kSlotsPerThread = HSK_MAX_HOT_SLOTS / kResolveThreads;

__device__ __forceinline__ bool is_claim(int32_t c) { return c <= INT_MIN + HSK_MAX_SELECTIONS_PER_REQUEST; }

__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(ResolveArgs a) {
  __shared__ uint32_t s_hit[HSK_MAX_HOT_SLOTS / 32];
  __shared__ uint32_t s_vic[HSK_MAX_HOT_SLOTS / 32];
  __shared__ int32_t s_hit_pre[HSK_MAX_HOT_SLOTS / 32];
  __shared__ int32_t s_vic_pre[HSK_MAX_HOT_SLOTS / 32];
  __shared__ uint16_t s_order[HSK_MAX_HOT_SLOTS];
  __shared__ uint16_t s_victim[HSK_MAX_HOT_SLOTS];
  __shared__ uint16_t s_neworder[HSK_MAX_HOT_SLOTS];
  __shared__ int s_wsum[2][kResolveWaves];
  __shared__ int s_cnt[4];

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int NT = kResolveThreads;
  const int64_t n = a.ctx[r];
  const int B = a.B;
  const int nwords = (B + 31) >> 5;
  const int total = a.Qmax * a.k;
  const int nq = a.nq ? a.nq[r] : a.Qmax;
  const bool nq_ok = nq >= 0 && nq <= a.Qmax;
  const int nsel = nq_ok ? nq * a.k : 0;
  const int32_t* sel = a.sel + (int64_t)r * total;
  int32_t* locs = a.locs + (int64_t)r * total;
  int32_t* key = a.m.key + (int64_t)r * B;
  uint32_t* rec = a.m.rec + (int64_t)r * B;
  uint16_t* order = a.m.order + (int64_t)r * B;
  int32_t* pt = a.m.pt + (int64_t)r * a.max_ctx;
  const int32_t* opt = a.m.opt ? a.m.opt + (int64_t)r * a.max_pages : nullptr;
  int32_t* ppos = a.m.plan_pos + (int64_t)r * a.plan_cap;
  int32_t* pdst = a.m.plan_dst + (int64_t)r * a.plan_cap;
  const int64_t hot0 = (int64_t)r * B;
  const int64_t stg0 = a.stg_base + (int64_t)r * a.S;
  // Stores count in the same in-order counter as loads on this architecture, so a load issued after a
  // burst of stores waits for all of them: every phase below does its loads before its stores, and the
  // metadata stores come last.
  constexpr int per_round = kResolveThreads * kPer;
  const int nrounds = (nsel + per_round - 1) / per_round;
  const bool one_round = nrounds <= 1;

  // ---- phase 0: slot order and keys to LDS, clear bitmaps, validate every selected position ------------
  // The selections are requested first: the page-table probes depend on them, and loads complete in order,
  // so the probes then wait for the selections only, not for the slot order and keys requested after them.
  bool bad = !nq_ok;
  int32_t pv[kPer];
  for (int rd = 0; rd < nrounds; ++rd) {
    const int fb = rd * per_round + kPer * tid;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int f = fb + e;
      pv[e] = f < nsel ? sel[f] : 0;
      bad |= (pv[e] < 0) || ((int64_t)pv[e] >= n);
    }
  }
  uint16_t ov_[kSlotsPerThread];
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int q = tid + j * NT;
    ov_[j] = q < B ? order[q] : 0;
  }
  for (int w = tid; w < nwords; w += NT) { s_hit[w] = 0u; s_vic[w] = 0u; }
  if (tid < 4) s_cnt[tid] = 0;
  // With one round, the page-table words (and optional-page map entries) of this thread's selections are
  // requested now, before the validation barrier, so the probe's latency overlaps it; positions are
  // clamped into the request's rows for the address only (an invalid request returns at the barrier).
  int32_t ptv[kPer], ovv[kPer];
  if (one_round) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int32_t pc = (pv[e] < 0 || n <= 0) ? 0 : ((int64_t)pv[e] >= n ? (int32_t)(n - 1) : pv[e]);
      ptv[e] = pt[pc];
      const int64_t page = opt ? min((int64_t)(pc / a.P), a.max_pages - 1) : 0;
      ovv[e] = opt ? opt[page] : -1;
    }
  }
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int q = tid + j * NT;
    if (q < B) s_order[q] = ov_[j];
  }
  int32_t* fill = a.fill ? a.fill + (int64_t)r * total : nullptr;
  // With a ready array (a copy kernel on another stream waits for this request's plan inside the kernel),
  // every exit publishes the plan: every wave waits until its stores are acknowledged by the L2, then, after
  // the barrier, one device-scope release (a single L2 write-back for the workgroup: one per wave made the
  // resolve four times slower beside a running attention) and the store of the call's epoch.  Every caller
  // below is reached by the whole workgroup.
  auto publish = [&]() {
    if (!a.ready) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(a.ready + r, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (__syncthreads_or(bad)) {
    for (int f = tid; f < total; f += NT) {
      locs[f] = -1;
      if (fill) fill[f] = -1;
    }
    if (tid == 0) {
      a.m.plan_n[r] = 0;
      if (a.stats) {
        hsk_stats z = {};
        z.status = HSK_ERANGE;
        a.stats[r] = z;
      }
      atomicCAS(a.err, 0, HSK_ERANGE);
    }
    publish();
    return;
  }

  // class counts and the request's statistics (every thread calls it): wave sums first (1,024 same-address
  // LDS atomics would serialise for microseconds), two counts per word in 16-bit fields (a wave handles at
  // most 64 x 4 x 16 = 4,096 selections), summed by the DPP scan and read from lane 63
  int my_tail = 0, my_opt = 0, my_hit_sel = 0, my_miss_sel = 0;
  auto write_stats = [&](int m_, int nhit_, int over_) {
    const int c01 = wave_incl_scan(my_tail | (my_opt << 16));
    const int c23 = wave_incl_scan(my_hit_sel | (my_miss_sel << 16));
    const int w01 = __builtin_amdgcn_readlane(c01, 63), w23 = __builtin_amdgcn_readlane(c23, 63);
    if ((tid & 63) == 0) {
      atomicAdd(&s_cnt[0], w01 & 0xFFFF);
      atomicAdd(&s_cnt[1], w01 >> 16);
      atomicAdd(&s_cnt[2], w23 & 0xFFFF);
      atomicAdd(&s_cnt[3], w23 >> 16);
    }
    lds_barrier();
    if (tid == 0) {
      a.m.plan_n[r] = m_;
      if (a.stats) {
        hsk_stats st;
        st.n_sel = nsel;
        st.n_tail = s_cnt[0];
        st.n_opt = s_cnt[1];
        st.n_hit = nhit_;
        st.n_hit_sel = s_cnt[2];
        st.n_miss = m_;
        st.n_miss_sel = s_cnt[3];
        st.n_staged = over_;
        st.status = HSK_OK;
        st.reserved = 0;
        st.fetched_bytes = (int64_t)m_ * a.row_bytes;
        a.stats[r] = st;
      }
    }
  };

  // ---- phase 1: direct pass, page-table probe, hit bitmap, first-occurrence claims of misses ----------
  // A missing position p gets atomicMin(pt[p], INT_MIN + f) from each selection f naming it, so the word
  // ends holding the first occurrence whatever the order of the atomics.
  int32_t code[kPer];
  for (int rd = 0; rd < nrounds; ++rd) {
    const int fb = rd * per_round + kPer * tid;
    if (!one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) pv[e] = fb + e < nsel ? sel[fb + e] : 0;
    }
    // branch-free loads, all issued before any is used: the page-table word (and the optional-page map
    // entry) of every selection, direct or not (with one round they were requested before the barrier)
    bool pend[kPer];
    if (!one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) ptv[e] = pt[pv[e]];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int64_t page = opt ? min((int64_t)(pv[e] / a.P), a.max_pages - 1) : 0;
        ovv[e] = opt ? opt[page] : -1;
      }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int f = fb + e;
      const int32_t p = pv[e];
      pend[e] = false;
      code[e] = -1;
      if (f < nsel) {
        if (p >= n - a.T) {
          ++my_tail;
          code[e] = (int32_t)((int64_t)a.R * a.B + (int64_t)r * a.T + (p % a.T));
        } else if (opt && (int64_t)(p / a.P) < n / a.P && ovv[e] >= 0) {
          ++my_opt;
          code[e] = (int32_t)(a.opt_base + (int64_t)ovv[e] * a.P + (p % a.P));
        } else {
          pend[e] = true;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (!pend[e]) continue;
      const int32_t s = ptv[e];
      if (s >= 0) {
        ++my_hit_sel;
        atomicOr(&s_hit[s >> 5], 1u << (s & 31));
        code[e] = (int32_t)(hot0 + s);
      } else {
        ++my_miss_sel;
        claim_min(&pt[pv[e]], INT_MIN + fb + e);
        code[e] = kCodeMiss;
      }
    }
    if (!one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (fb + e < nsel) locs[fb + e] = code[e];
    }
  }

  // ---- no miss in this request: no claims, victims or copies.  The slot order becomes [slots not hit, in
  // their old order][hit slots ascending], which is the ascending (rec, slot) order once the hits get 2e + 1;
  // one block scan ranks both groups (two counts per word in 16-bit fields: at most B <= 8,192 each).
  // Every location is final already (a direct row or a hit's slot).
  if (!__syncthreads_or(my_miss_sel != 0)) {
    const int per = (B + NT - 1) / NT;
    const int q0 = tid * per;
    uint16_t sl[kSlotsPerThread];
    int cnt_nh = 0;
#pragma unroll
    for (int e = 0; e < kSlotsPerThread; ++e) {
      sl[e] = 0xFFFF;
      if (e < per && q0 + e < B) {
        const int sv = s_order[q0 + e];
        if (((s_hit[sv >> 5] >> (sv & 31)) & 1u) == 0u) { sl[e] = (uint16_t)sv; ++cnt_nh; }
      }
    }
    const int hw = tid < nwords ? __popc(s_hit[tid]) : 0;
    int tot;
    const int pre = block_sum_scan(cnt_nh | (hw << 16), &tot, s_wsum[0]);
    const int n_nonhit = tot & 0xFFFF, nhit0 = tot >> 16;
    if (tid < nwords) s_hit_pre[tid] = pre >> 16;
    int rank = pre & 0xFFFF;
#pragma unroll
    for (int e = 0; e < kSlotsPerThread; ++e)
      if (sl[e] != 0xFFFF) order[rank++] = sl[e];
    lds_barrier();
    const uint32_t e2h = 2u * a.epoch + 1u;
    for (int sv = tid; sv < B; sv += NT) {
      const int w = sv >> 5;
      const uint32_t bit = 1u << (sv & 31);
      if (s_hit[w] & bit) {
        order[n_nonhit + s_hit_pre[w] + __popc(s_hit[w] & (bit - 1u))] = (uint16_t)sv;
        rec[sv] = e2h;
      }
    }
    if (one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (kPer * tid + e < nsel) locs[kPer * tid + e] = code[e];
    }
    for (int f = nsel + tid; f < total; f += NT) locs[f] = -1;
    if (fill)
      for (int f = tid; f < total; f += NT) fill[f] = -1;
    write_stats(0, nhit0, 0);
    publish();
    return;
  }

  // ---- phase 2: distinct misses in first-occurrence order (ascending f) --------------------------------
  int m = 0;
  for (int rd = 0; rd < nrounds; ++rd) {
    const int fb = rd * per_round + kPer * tid;
    if (!one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        code[e] = fb + e < nsel ? locs[fb + e] : -1;
        pv[e] = fb + e < nsel ? sel[fb + e] : 0;
      }
    }
    bool first[kPer];
    int nfirst = 0;
    int32_t cv[kPer];
    // only missing selections hold a claim to read back (all issued together; hits and direct rows skip)
#pragma unroll
    for (int e = 0; e < kPer; ++e) cv[e] = (fb + e < nsel && code[e] == kCodeMiss) ? rmw_read(&pt[pv[e]]) : 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      first[e] = false;
      if (fb + e < nsel && code[e] == kCodeMiss) {
        first[e] = cv[e] == INT_MIN + fb + e;
        if (!first[e]) code[e] = cv[e];  // a repeat keeps the claim, i.e. its first occurrence
        nfirst += first[e];
      }
    }
    if (fill) {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (fb + e < nsel)
          fill[fb + e] = (code[e] == kCodeMiss || is_claim(code[e])) ? 2 * pv[e] + (first[e] ? 1 : 0) : -1;
    }
    int cnt;
    int idx = m + block_sum_scan(nfirst, &cnt, s_wsum[rd & 1]);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (first[e]) {
        ppos[idx] = pv[e];
        code[e] = -2 - idx;
        locs[fb + e] = code[e];
        ++idx;
      } else if (!one_round && fb + e < nsel) {
        locs[fb + e] = code[e];
      }
    }
    m += cnt;
  }
  __syncthreads();
  // repeats of a miss look up their first occurrence's miss index now, before the stores of the next phases
  for (int rd = 0; rd < nrounds; ++rd) {
    const int fb = rd * per_round + kPer * tid;
    if (!one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) code[e] = fb + e < nsel ? locs[fb + e] : -1;
    }
    bool rep = false;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (fb + e < nsel && is_claim(code[e])) {
        code[e] = rmw_read(&locs[code[e] - INT_MIN]);
        rep = true;
      }
    }
    if (!one_round && rep) {
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (fb + e < nsel) locs[fb + e] = code[e];
    }
  }

  // the first two strided miss entries this thread will fill, read before the stores of phases 4 and 5
  const int32_t pp0 = tid < m ? ppos[tid] : 0;
  const int32_t pp1 = tid + NT < m ? ppos[tid + NT] : 0;

  // ---- phase 3: hit count, staging overflow check, victims over the slot order -----------------------
  int nhit = 0;
  {
    const int hw = tid < nwords ? __popc(s_hit[tid]) : 0;
    const int pre = block_sum_scan(hw, &nhit, s_wsum[0]);
    if (tid < nwords) s_hit_pre[tid] = pre;
  }
  const int free_slots = B - nhit;
  const int v = m < free_slots ? m : free_slots;
  const int over = m - v;
  if (over > a.S) {
    for (int i = tid; i < m; i += NT) pt[ppos[i]] = -1;  // drop the claims
    for (int f = tid; f < total; f += NT) {
      locs[f] = -1;
      if (fill) fill[f] = -1;
    }
    if (tid == 0) {
      a.m.plan_n[r] = 0;
      if (a.stats) {
        hsk_stats z = {};
        z.status = HSK_ESTAGE;
        a.stats[r] = z;
      }
      atomicCAS(a.err, 0, HSK_ESTAGE);
    }
    publish();
    return;
  }
  const int n_keep = free_slots - v;
  {
    // thread t walks order positions [t * per, t * per + per): one block scan ranks every non-hit slot
    const int per = (B + NT - 1) / NT;
    const int q0 = tid * per;
    uint16_t sl[kSlotsPerThread];
    int cnt_nh = 0;
#pragma unroll
    for (int e = 0; e < kSlotsPerThread; ++e) {
      sl[e] = 0xFFFF;
      if (e < per && q0 + e < B) {
        const int s = s_order[q0 + e];
        if (((s_hit[s >> 5] >> (s & 31)) & 1u) == 0u) { sl[e] = (uint16_t)s; ++cnt_nh; }
      }
    }
    int tot;
    int rank = block_sum_scan(cnt_nh, &tot, s_wsum[1]);
#pragma unroll
    for (int e = 0; e < kSlotsPerThread; ++e) {
      if (sl[e] == 0xFFFF) continue;
      const int s = sl[e];
      if (rank < v) {
        s_victim[rank] = (uint16_t)s;
        atomicOr(&s_vic[s >> 5], 1u << (s & 31));
      } else {
        s_neworder[rank - v] = (uint16_t)s;  // unselected non-victims keep their relative order
      }
      ++rank;
    }
  }
  __syncthreads();
  {
    const int vw = tid < nwords ? __popc(s_vic[tid]) : 0;
    int vtot;
    const int pre = block_sum_scan(vw, &vtot, s_wsum[0]);
    if (tid < nwords) s_vic_pre[tid] = pre;
  }
  __syncthreads();
  // the positions held by the first two strided victims this thread evicts, read before the stores of phases 4
  // and 5 (later victims, past 2,048 per request, are read where they are evicted)
  const int32_t old0 = tid < v ? key[s_victim[tid]] : -1;
  const int32_t old1 = tid + NT < v ? key[s_victim[tid + NT]] : -1;

  // ---- phase 4: publish locations in selection order ---------------------------------------------------
  for (int rd = 0; rd < nrounds; ++rd) {
    const int fb = rd * per_round + kPer * tid;
    if (!one_round) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) code[e] = fb + e < nsel ? locs[fb + e] : -1;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int f = fb + e;
      if (f >= nsel) continue;
      const int32_t c = code[e];
      int32_t loc;
      if (c >= 0) {
        loc = c;
      } else {
        const int i = -2 - c;
        loc = i < v ? (int32_t)(hot0 + s_victim[i]) : (int32_t)(stg0 + (i - v));
      }
      locs[f] = loc;
    }
  }
  for (int f = nsel + tid; f < total; f += NT) {
    locs[f] = -1;
    if (fill) fill[f] = -1;
  }

  // ---- phase 5: metadata update -- fills (2e) then hits (2e+1) at the most recent end ------------------
  const uint32_t e2 = 2u * a.epoch;
  for (int s = tid; s < B; s += NT) {
    const int w = s >> 5;
    const uint32_t bit = 1u << (s & 31), below = bit - 1u;
    if (s_vic[w] & bit) {
      s_neworder[n_keep + s_vic_pre[w] + __popc(s_vic[w] & below)] = (uint16_t)s;
    } else if (s_hit[w] & bit) {
      s_neworder[n_keep + v + s_hit_pre[w] + __popc(s_hit[w] & below)] = (uint16_t)s;
      rec[s] = e2 + 1u;
    }
  }
  for (int i = tid; i < m; i += NT) {
    const int32_t p = i == tid ? pp0 : i == tid + NT ? pp1 : ppos[i];
    if (i < v) {
      const int s = s_victim[i];
      const int32_t old = i == tid ? old0 : i == tid + NT ? old1 : key[s];
      if (old >= 0) pt[old] = -1;  // eviction: old is not pending in this call
      key[s] = p;
      rec[s] = e2;
      pt[p] = s;
      pdst[i] = (int32_t)(hot0 + s);
    } else {
      pt[p] = -1;  // staged rows stay outside the hot cache
      pdst[i] = (int32_t)(stg0 + (i - v));
    }
  }
  lds_barrier();
  for (int q = tid; q < B; q += NT) order[q] = s_neworder[q];
  write_stats(m, nhit, over);

  // ---- phase 6: this call's distinct missing rows, host -> pool ------------------------------------------
  // The copy done by GPU threads (HiSparse section 3.4, phase 4), here by the resolving workgroup itself, so
  // a resolve is one launch: zero-copy 16-byte loads of the pinned host rows over PCIe.  Wave w copies miss
  // rows 4 w .. 4 w + 3, then the four rows kResolveWaves * 4 further on, and so on; a batch's positions are
  // read first (written by phase 2 before this workgroup's barriers), then every chunk of the batch is loaded
  // before any is stored.  Each of a workgroup's 16 waves keeps up to four rows' reads in flight (64 requests
  // of 1,152-byte rows: ~4.7 MB), far more than the link needs to stream.
  if (a.host != nullptr && m > 0) {
    const int lane = tid & 63, wv = tid >> 6;
    const int cpr = a.row_bytes >> 4;  // 16-byte chunks per row
    const char* hreq = a.host + (int64_t)r * a.host_req_stride;
    for (int i0 = 4 * wv; i0 < m; i0 += 4 * kResolveWaves) {
      const u32x4* src[4];
      u32x4* dst[4];
      int nrow = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u;
        const bool ok = i < m;
        const int32_t p = ok ? ppos[i] : 0;
        const int64_t d = !ok ? 0 : (i < v ? hot0 + s_victim[i] : stg0 + (i - v));
        src[u] = (const u32x4*)(hreq + (int64_t)p * a.row_bytes);
        dst[u] = (u32x4*)(a.pool + d * a.row_bytes);
        nrow += ok;
      }
      for (int c0 = 0; c0 < cpr; c0 += 128) {
        u32x4 buf[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = c0 + 64 * h + lane;
            if (u < nrow && c < cpr) buf[u][h] = __builtin_nontemporal_load(src[u] + c);
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = c0 + 64 * h + lane;
            if (u < nrow && c < cpr) dst[u][c] = buf[u][h];
          }
      }
    }
  }
  publish();
}


// Copy one row of `chunks` 16-byte chunks with the 64 lanes of a wave: all loads first, then stores.
__device__ __forceinline__ void wave_copy_row(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int chunks,
                                              int lane) {
  constexpr int kDepth = 8;
  for (int c0 = 0; c0 < chunks; c0 += 64 * kDepth) {
    u32x4 buf[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int c = c0 + d * 64 + lane;
      if (c < chunks) buf[d] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int c = c0 + d * 64 + lane;
      if (c < chunks) dst[c] = buf[d];
    }
  }
}

// Host -> device gather of a miss plan (HiSparse section 3.4 phase 4, the copy done by GPU threads; section 3.5
// replay): 16-byte zero-copy loads from pinned host memory over PCIe into the pool rows.
// Rows are numbered globally in request order (rows of earlier requests first) and wave w of the 1-D grid
// copies the rows whose number is w modulo the number of waves, so every wave gets the same share however
// the misses are spread over requests.  A wave first lists its rows (host and pool addresses) in LDS, 64
// requests at a time with one request per lane, then copies the listed rows as one stream of 16-byte chunks
// over its 64 lanes, kDepth loads in flight per lane before the stores.
constexpr int kGatherWaves = kFetchThreads / 64;
constexpr int kGatherList = 64;

// Promotion copy-back ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", section 3.4
// and Figure 3 callout 3: promoted staged rows are copied back to stable hot-cache addresses before the staging
// arena is reused).  Reading: queries 0..A of a request (the anchor and its A accepted drafts) are committed;
// the staged rows of the last resolve that a committed query selected (in staging order, skipping rows already
// hot) take the hot slots touched at that epoch whose rows no committed query selected, in ascending
// (rec, slot) order -- the slot order list -- and become fills of the epoch (rec = 2e).  One 1024-thread
// workgroup per request:
//   1. committed selections mark their hot slots and staging rows in two LDS bitmaps (from the locations the
//      resolve emitted);
//   2. the marked staging rows not yet hot are compacted in staging order (block prefix sum); a marked row
//      that is already hot (promoted by an earlier call after the same resolve) marks its slot instead;
//   3. the unmarked slots of this epoch are compacted in slot-order-list order;
//   4. pair i takes slot D_i for staged row P_i: page table, key and recency updated;
//   5. the slot order is rewritten: its prefix of older slots is unchanged, then this epoch's fills, then its
//      hits, each by ascending slot (the promoted slots count as fills);
//   6. the rows are copied from their staging rows into the slots' pool rows.
struct PromoteArgs {
  const int32_t* locs;
  const int32_t* nq;
  const int32_t* accepted;
  int32_t* promoted;
  SourceMeta m;
  char* pool;
  int64_t max_ctx;
  int64_t stg_base;
  int32_t R, B, S, Qmax, k, row_bytes;
  uint32_t epoch;
};

__global__ __launch_bounds__(kResolveThreads) void promote_kernel(PromoteArgs a) {
  __shared__ uint32_t s_hot[HSK_MAX_HOT_SLOTS / 32];                 // committed hot slots
  __shared__ uint32_t s_dem[HSK_MAX_HOT_SLOTS / 32];                 // slots that receive a promoted row
  __shared__ uint32_t s_stg[HSK_MAX_SELECTIONS_PER_REQUEST / 32];    // staging rows a committed query selected
  __shared__ uint16_t s_P[HSK_MAX_HOT_SLOTS];                        // promotable staging rows, in order
  __shared__ uint16_t s_D[HSK_MAX_HOT_SLOTS];                        // demotable slots, in order
  __shared__ int s_wsum[2][kResolveWaves];
  __shared__ int s_v;
  const int r = blockIdx.x, tid = threadIdx.x, NT = kResolveThreads;
  const int B = a.B, S = a.S;
  const int nq = a.nq ? a.nq[r] : a.Qmax;
  if (nq <= 0 || nq > a.Qmax) {
    if (a.promoted && tid == 0) a.promoted[r] = 0;
    return;
  }
  const int A = min(max(a.accepted[r], 0), nq - 1);
  const int32_t* locs = a.locs + (int64_t)r * a.Qmax * a.k;
  int32_t* key = a.m.key + (int64_t)r * B;
  uint32_t* rec = a.m.rec + (int64_t)r * B;
  uint16_t* order = a.m.order + (int64_t)r * B;
  int32_t* pt = a.m.pt + (int64_t)r * a.max_ctx;
  const int32_t* ppos = a.m.plan_pos + (int64_t)r * a.Qmax * a.k;
  const int32_t* pdst = a.m.plan_dst + (int64_t)r * a.Qmax * a.k;
  const int plan_n = a.m.plan_n[r];
  const int64_t hot0 = (int64_t)r * B, stg0 = a.stg_base + (int64_t)r * S;
  const uint32_t e2 = 2u * a.epoch;
  const int bw = (B + 31) >> 5, sw = (S + 31) >> 5;
  for (int w = tid; w < bw; w += NT) { s_hot[w] = 0u; s_dem[w] = 0u; }
  for (int w = tid; w < sw; w += NT) s_stg[w] = 0u;
  if (tid == 0) s_v = plan_n;
  __syncthreads();
  // 1. marks from the committed queries' locations; v = the first staged entry of the plan (fills come first)
  const int ncommit = (A + 1) * a.k;
  for (int f = tid; f < ncommit; f += NT) {
    const int64_t loc = locs[f];
    if (loc >= hot0 && loc < hot0 + B) atomicOr(&s_hot[(loc - hot0) >> 5], 1u << ((loc - hot0) & 31));
    else if (loc >= stg0 && loc < stg0 + S) atomicOr(&s_stg[(loc - stg0) >> 5], 1u << ((loc - stg0) & 31));
  }
  for (int i = tid; i < plan_n; i += NT)
    if (pdst[i] >= stg0 && pdst[i] < stg0 + S) atomicMin(&s_v, i);
  __syncthreads();
  const int v = s_v;
  // 2. promotable staging rows in staging order; thread t owns rows [t * per, (t + 1) * per)
  const int per = (S + NT - 1) / NT;
  int cnt = 0;
  // (a staging row is taken only if the plan lists it, so locations that do not come from the source's last
  // resolve cannot index past the plan or the page table)
  auto staged_pos = [&](int c) -> int32_t {
    if (!((s_stg[c >> 5] >> (c & 31)) & 1u) || v + c >= plan_n) return -1;
    const int32_t u = ppos[v + c];
    return (u >= 0 && u < a.max_ctx) ? u : -1;
  };
  for (int c = tid * per; c < min(S, (tid + 1) * per); ++c) {
    const int32_t u = staged_pos(c);
    if (u < 0) continue;
    const int32_t slot = pt[u];
    if (slot >= 0 && slot < B) atomicOr(&s_hot[slot >> 5], 1u << (slot & 31));   // promoted earlier: committed, hot
    else ++cnt;
  }
  int np;
  int base = block_sum_scan(cnt, &np, s_wsum[0]);
  for (int c = tid * per; c < min(S, (tid + 1) * per) && base < B; ++c) {
    const int32_t u = staged_pos(c);
    if (u < 0 || pt[u] >= 0) continue;
    s_P[base++] = (uint16_t)c;
  }
  __syncthreads();
  // 3. demotable slots in slot-order-list order: touched at this epoch, holding a row no committed query chose
  const int pers = (B + NT - 1) / NT;
  int dcnt = 0;
  for (int i = tid * pers; i < min(B, (tid + 1) * pers); ++i) {
    const int slot = order[i];
    dcnt += (rec[slot] >= e2 && key[slot] >= 0 && key[slot] < a.max_ctx && !((s_hot[slot >> 5] >> (slot & 31)) & 1u)) ? 1 : 0;
  }
  int nd;
  int dbase = block_sum_scan(dcnt, &nd, s_wsum[1]);
  for (int i = tid * pers; i < min(B, (tid + 1) * pers); ++i) {
    const int slot = order[i];
    if (rec[slot] >= e2 && key[slot] >= 0 && key[slot] < a.max_ctx && !((s_hot[slot >> 5] >> (slot & 31)) & 1u))
      s_D[dbase++] = (uint16_t)slot;
  }
  np = min(np, B);
  const int m = min(np, nd);
  __syncthreads();
  // 4. metadata of the pairs (distinct old and new positions, distinct slots)
  for (int i = tid; i < m; i += NT) {
    const int slot = s_D[i];
    const int32_t u = ppos[v + s_P[i]];
    pt[key[slot]] = -1;
    key[slot] = u;
    pt[u] = slot;
    rec[slot] = e2;
    atomicOr(&s_dem[slot >> 5], 1u << (slot & 31));
  }
  __syncthreads();
  // 5. slot order: [slots older than this epoch, unchanged prefix][fills of the epoch][hits], by slot
  int old_n = 0, fill_n = 0, hit_n = 0;
  bool is_fill[kSlotsPerThread], is_hit[kSlotsPerThread];
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int slot = tid * kSlotsPerThread + j;
    is_fill[j] = is_hit[j] = false;
    if (slot < B) {
      const uint32_t rc = rec[slot];
      const bool dem = (s_dem[slot >> 5] >> (slot & 31)) & 1u;
      is_fill[j] = rc == e2 || dem;
      is_hit[j] = rc == e2 + 1u && !dem;
      old_n += rc < e2 ? 1 : 0;
      fill_n += is_fill[j] ? 1 : 0;
      hit_n += is_hit[j] ? 1 : 0;
    }
  }
  int n_old, n_fill, n_hit;
  const int fbase = block_sum_scan(fill_n, &n_fill, s_wsum[0]);
  const int hbase = block_sum_scan(hit_n, &n_hit, s_wsum[1]);
  (void)block_sum_scan(old_n, &n_old, s_wsum[0]);
  __syncthreads();
  int fi = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int slot = tid * kSlotsPerThread + j;
    if (is_fill[j]) order[n_old + fbase + fi++] = (uint16_t)slot;
    if (is_hit[j]) order[n_old + n_fill + hbase + hi++] = (uint16_t)slot;
  }
  // 6. copy the promoted rows from staging into their slots, 16 bytes per lane, one row per wave at a time
  const int lane = tid & 63, wave = tid >> 6;
  const int chunks = a.row_bytes >> 4;
  for (int i = wave; i < m; i += kResolveWaves) {
    const u32x4* src = (const u32x4*)(a.pool + (stg0 + s_P[i]) * (int64_t)a.row_bytes);
    u32x4* dst = (u32x4*)(a.pool + (hot0 + s_D[i]) * (int64_t)a.row_bytes);
    for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
  }
  if (a.promoted && tid == 0) a.promoted[r] = m;
}

__global__ __launch_bounds__(kFetchThreads) void gather_kernel(GatherArgs g, int32_t R) {
  __shared__ const char* s_src[kGatherWaves][kGatherList];
  __shared__ char* s_dst[kGatherWaves][kGatherList];
  constexpr int kDepth = 4;  // 16-byte loads in flight per lane (fewer or more slowed the overlapped step)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kGatherWaves;
  const int64_t gw = (int64_t)blockIdx.x * kGatherWaves + wave;
  const int cpr = g.row_bytes >> 4;  // 16-byte chunks per row
  const uint64_t below = (1ull << lane) - 1ull;
  int nl = 0;

  auto flush = [&]() {
    const int total = nl * cpr;
    for (int x0 = 0; x0 < total; x0 += 64 * kDepth) {
      u32x4 buf[kDepth];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int x = x0 + d * 64 + lane;
        if (x < total) {
          const int row = x / cpr;
          buf[d] = __builtin_nontemporal_load((const u32x4*)s_src[wave][row] + (x - row * cpr));
        }
      }
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int x = x0 + d * 64 + lane;
        if (x < total) {
          const int row = x / cpr;
          ((u32x4*)s_dst[wave][row])[x - row * cpr] = buf[d];
        }
      }
    }
    nl = 0;
  };

  int64_t C = 0;  // rows of the requests before this group of 64
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int r = r0 + lane;
    bool ok = true;
    if (g.ready) {
      // request r's plan comes from a resolve on another stream: wait (bounded) until it publishes this
      // call's epoch, then acquire; a plan that never appears is an error and its request copies nothing
      ok = r >= R;
      for (uint32_t spin = 0; !ok; ++spin) {
        ok = __hip_atomic_load(g.ready + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g.epoch;
        if (ok) break;
        if (spin >= kPlanSpinLimit) {
          atomicCAS(g.err, 0, HSK_ESTATE);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    const int m = r < R && ok ? g.plan_n[r] : 0;
    int64_t incl = m;  // inclusive prefix over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int64_t Cr = C + incl - m;
    const int64_t i0 = ((gw - Cr) % nw + nw) % nw;  // first row of request r that falls to this wave
    const int cnt = i0 < m ? (int)((m - 1 - i0) / nw + 1) : 0;
    const char* hbase = g.host + (int64_t)r * g.host_req_stride;
    const int32_t* pp = g.plan_pos + (int64_t)r * g.plan_cap;
    const int32_t* pd = g.plan_dst + (int64_t)r * g.plan_cap;
    for (int k = 0; __ballot(k < cnt); ++k) {
      const bool has = k < cnt;
      const uint64_t mask = __ballot(has);
      const int nnew = __popcll(mask);
      if (nl + nnew > kGatherList) flush();
      if (has) {
        const int slot = nl + __popcll(mask & below);
        const int64_t i = i0 + (int64_t)k * nw;
        s_src[wave][slot] = hbase + (int64_t)pp[i] * g.row_bytes;
        s_dst[wave][slot] = g.pool + (int64_t)pd[i] * g.row_bytes;
      }
      nl += nnew;
    }
    C += __shfl(incl, 63, 64);
  }
  if (nl) flush();
}

// Tail rows [n_r - T, n_r) of every request: host -> pool row R*B + r*T + (p mod T).
__global__ __launch_bounds__(kGatherThreads) void tail_copy_kernel(const char* host, int64_t stride, char* pool,
                                                                   const int64_t* ctx, int32_t R, int32_t B,
                                                                   int32_t T, int32_t row_bytes) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kWaves = kGatherThreads / 64;
  const int64_t n = ctx[r];
  for (int t = blockIdx.x * kWaves + wave; t < T; t += gridDim.x * kWaves) {
    const int64_t p = n - T + t;
    if (p < 0) continue;
    const u32x4* src = (const u32x4*)(host + r * stride + p * row_bytes);
    u32x4* dst = (u32x4*)(pool + ((int64_t)R * B + (int64_t)r * T + (p % T)) * row_bytes);
    wave_copy_row(src, dst, row_bytes >> 4, lane);
  }
}

// Decode-loop append (HiSparse section 3.3 step 4; Adaptive DHiSparse section 3.2): one block per request
// copies its `count` new rows into the tail ring (row R*B + r*T + (p mod T) for p = n_r, ..), records n_r for
// the write-through and advances n_r.
__global__ __launch_bounds__(kGatherThreads) void append_tail_kernel(const char* rows, char* pool, int64_t* ctx,
                                                                     int32_t* wt_pos, int32_t R, int32_t B,
                                                                     int32_t T, int32_t count, int32_t row_bytes) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kWaves = kGatherThreads / 64;
  const int64_t n = ctx[r];
  if (n < 0) {  // a free slot (scheduled residency): nothing appended, nothing written through
    if (threadIdx.x == 0) wt_pos[r] = -1;
    return;
  }
  for (int i = wave; i < count; i += kWaves) {
    const u32x4* src = (const u32x4*)(rows + ((int64_t)r * count + i) * row_bytes);
    u32x4* dst = (u32x4*)(pool + ((int64_t)R * B + (int64_t)r * T + ((n + i) % T)) * row_bytes);
    wave_copy_row(src, dst, row_bytes >> 4, lane);
  }
  __syncthreads();  // every thread has read n_r
  if (threadIdx.x == 0) {
    wt_pos[r] = (int32_t)n;
    ctx[r] = n + count;
  }
}

// Write-through of an append: tail ring rows of positions wt_pos[r] .. + count - 1 -> the request's pinned
// host rows (device stores over the host link).
__global__ __launch_bounds__(kGatherThreads) void write_through_kernel(const char* pool, char* host, int64_t stride,
                                                                       const int32_t* wt_pos, int32_t R, int32_t B,
                                                                       int32_t T, int32_t count,
                                                                       int32_t row_bytes) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kWaves = kGatherThreads / 64;
  const int64_t p0 = wt_pos[r];
  if (p0 < 0) return;  // free slot
  for (int i = wave; i < count; i += kWaves) {
    const u32x4* src = (const u32x4*)(pool + ((int64_t)R * B + (int64_t)r * T + ((p0 + i) % T)) * row_bytes);
    u32x4* dst = (u32x4*)(host + r * stride + (p0 + i) * row_bytes);
    wave_copy_row(src, dst, row_bytes >> 4, lane);
  }
}

// Draft ring (Adaptive DHiSparse Eqs. 9-10): one block per slot writes its `count` new rows to i*R_d + (t mod R_d).
__global__ __launch_bounds__(kGatherThreads) void ring_write_kernel(char* ring, int64_t ring_rows, const char* rows,
                                                                    int32_t count, int32_t row_bytes,
                                                                    const int64_t* t0) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kWaves = kGatherThreads / 64;
  const int64_t t = t0[i];
  for (int j = wave; j < count; j += kWaves) {
    const u32x4* src = (const u32x4*)(rows + ((int64_t)i * count + j) * row_bytes);
    u32x4* dst = (u32x4*)(ring + ((int64_t)i * ring_rows + (t + j) % ring_rows) * row_bytes);
    wave_copy_row(src, dst, row_bytes >> 4, lane);
  }
}

__global__ void ring_locs_kernel(int64_t ring_rows, int32_t slots, int32_t window, const int64_t* t_end,
                                 int32_t* locs) {
  const int64_t n = (int64_t)slots * window;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = x / window, j = x % window;
    const int64_t t = t_end[i] - window + j;
    locs[x] = t < 0 ? -1 : (int32_t)(i * ring_rows + t % ring_rows);
  }
}

// Contiguous byte runs host -> pool (optional-history population); one block per run.
__global__ __launch_bounds__(kGatherThreads) void copy_runs_kernel(const char* host, char* pool, const CopyRun* runs) {
  const CopyRun run = runs[blockIdx.x];
  const u32x4* src = (const u32x4*)(host + run.src);
  u32x4* dst = (u32x4*)(pool + run.dst);
  const int64_t chunks = run.bytes >> 4;
  for (int64_t c = threadIdx.x; c < chunks; c += kGatherThreads) dst[c] = __builtin_nontemporal_load(src + c);
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void init_order_kernel(uint16_t* order, uint32_t* rec, int64_t total, int32_t B) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    order[i] = (uint16_t)(i % B);
    rec[i] = 0u;
  }
}

static unsigned grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_init_meta(const SourceMeta& m, int32_t R, int32_t B, int64_t max_ctx, int64_t max_pages,
                            hipStream_t s) {
  hipError_t e;
  if ((e = launch_fill_i32(m.key, (int64_t)R * B, -1, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(init_order_kernel, dim3(grid_for((int64_t)R * B, 256)), dim3(256), 0, s, m.order, m.rec,
                     (int64_t)R * B, B);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_fill_i32(m.pt, (int64_t)R * max_ctx, -1, s)) != hipSuccess) return e;
  if (m.opt && (e = launch_fill_i32(m.opt, (int64_t)R * max_pages, -1, s)) != hipSuccess) return e;
  if ((e = launch_fill_i32(m.plan_n, R, 0, s)) != hipSuccess) return e;
  return launch_fill_i32((int32_t*)m.ready, R, 0, s);  // epochs start at 1: no plan published yet
}

hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(resolve_kernel, dim3(a.R), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_promote(const int32_t* locs, const int32_t* nq, const int32_t* accepted, int32_t* promoted,
                          const SourceMeta& m, char* pool, int64_t max_ctx, int64_t stg_base, int32_t R, int32_t B,
                          int32_t S, int32_t Qmax, int32_t k, int32_t row_bytes, uint32_t epoch, hipStream_t s) {
  PromoteArgs a;
  a.locs = locs; a.nq = nq; a.accepted = accepted; a.promoted = promoted; a.m = m; a.pool = pool;
  a.max_ctx = max_ctx; a.stg_base = stg_base; a.R = R; a.B = B; a.S = S; a.Qmax = Qmax; a.k = k;
  a.row_bytes = row_bytes; a.epoch = epoch;
  hipLaunchKernelGGL(promote_kernel, dim3(R), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}

// done: an event that the launch itself records when the kernel ends (its completion signal), so no separate
// marker follows the kernel on its stream
hipError_t launch_gather(const GatherArgs& g, int32_t R, int32_t blocks, hipStream_t s, hipEvent_t done) {
  if (done) {
    hipExtLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(kFetchThreads), 0, s, nullptr, done, 0u, g, R);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(kFetchThreads), 0, s, g, R);
  return hipGetLastError();
}

hipError_t launch_tail_copy(const char* host, int64_t stride, char* pool, const int64_t* d_ctx, int32_t R,
                            int32_t B, int32_t T, int32_t row_bytes, hipStream_t s) {
  const int blocks = (T + 3) / 4 < 64 ? (T + 3) / 4 : 64;
  hipLaunchKernelGGL(tail_copy_kernel, dim3(blocks > 0 ? blocks : 1, R), dim3(kGatherThreads), 0, s, host, stride,
                     pool, d_ctx, R, B, T, row_bytes);
  return hipGetLastError();
}

hipError_t launch_append_tail(const char* rows, char* pool, int64_t* ctx, int32_t* wt_pos, int32_t R, int32_t B,
                              int32_t T, int32_t count, int32_t row_bytes, hipStream_t s) {
  hipLaunchKernelGGL(append_tail_kernel, dim3(R), dim3(kGatherThreads), 0, s, rows, pool, ctx, wt_pos, R, B, T, count,
                     row_bytes);
  return hipGetLastError();
}

hipError_t launch_write_through(const char* pool, char* host, int64_t stride, const int32_t* wt_pos, int32_t R,
                                int32_t B, int32_t T, int32_t count, int32_t row_bytes, hipStream_t s) {
  hipLaunchKernelGGL(write_through_kernel, dim3(R), dim3(kGatherThreads), 0, s, pool, host, stride, wt_pos, R, B, T,
                     count, row_bytes);
  return hipGetLastError();
}

hipError_t launch_ring_write(char* ring, int64_t ring_rows, int32_t slots, const char* rows, int32_t count,
                             int32_t row_bytes, const int64_t* t0, hipStream_t s) {
  hipLaunchKernelGGL(ring_write_kernel, dim3(slots), dim3(kGatherThreads), 0, s, ring, ring_rows, rows, count,
                     row_bytes, t0);
  return hipGetLastError();
}

hipError_t launch_ring_locs(int64_t ring_rows, int32_t slots, int32_t window, const int64_t* t_end, int32_t* locs,
                            hipStream_t s) {
  hipLaunchKernelGGL(ring_locs_kernel, dim3(grid_for((int64_t)slots * window, 256)), dim3(256), 0, s, ring_rows,
                     slots, window, t_end, locs);
  return hipGetLastError();
}

hipError_t launch_copy_runs(const char* host, char* pool, const CopyRun* runs, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_runs_kernel, dim3(n), dim3(kGatherThreads), 0, s, host, pool, runs);
  return hipGetLastError();
}

}  // namespace hsk
