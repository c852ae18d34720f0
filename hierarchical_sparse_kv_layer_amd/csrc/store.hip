// Host runtime of libhsk.so: store lifetime, workspace layout, residency, resolve/attention entry points.
//
// Data layout in HBM (caller-owned):
//   workspace: per request context lengths, a sticky error word, the per-selection host sources of a fused
//              resolve + attend [R][Qmax][k] i32, then per source
//              key[R][B] i32, rec[R][B] u32, order[R][B] u16, pt[R][max_ctx] i32, opt[R][max_pages] i32,
//              plan_n[R] i32, plan_pos[R][Qmax*k] i32, plan_dst[R][Qmax*k] i32, ready[R] u32 (each region
//              256-B aligned)
//   pool:      per source rows_per_source rows of row_bytes: [R*B hot | R*T tail | optional pages | R*S staging]
// Host (library-owned, pinned and mapped): per host source R x max_ctx rows of row_bytes.
#include <algorithm>
#include <cstring>
#include <new>

#include "hsk_internal.h"

namespace hsk {

static int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t total_pool_rows(const hsk_desc& d) {
  return rows_per_source(d) * d.num_sources +
         (d.staging_arenas ? (int64_t)d.staging_arenas * d.num_requests * d.staging_rows : 0);
}

// first staging row of a source, relative to the source's region
int64_t stg_base_of(const hsk_desc& d, int32_t source) {
  const int64_t R = d.num_requests;
  if (!d.staging_arenas) return R * d.hot_slots + R * d.tail_rows + d.opt_pool_pages * d.page_rows;
  const int64_t P = rows_per_source(d);
  return P * d.num_sources + (int64_t)(source % d.staging_arenas) * R * d.staging_rows - (int64_t)source * P;
}

// rows of one source region (staging included only without shared arenas)
int64_t rows_per_source(const hsk_desc& d) {
  return (int64_t)d.num_requests * d.hot_slots + (int64_t)d.num_requests * d.tail_rows +
         d.opt_pool_pages * d.page_rows + (d.staging_arenas ? 0 : (int64_t)d.num_requests * d.staging_rows);
}

static bool valid_desc(const hsk_desc* d) {
  if (!d) return false;
  if (d->num_requests < 1 || d->num_sources < 1) return false;
  if (d->row_bytes <= 0 || d->row_bytes % 16 != 0) return false;
  if (d->hot_slots < 1 || d->hot_slots > HSK_MAX_HOT_SLOTS) return false;
  if (d->tail_rows < 0 || d->page_rows < 0 || d->opt_pool_pages < 0 || d->staging_rows < 0) return false;
  if (d->page_rows == 0 && d->opt_pool_pages != 0) return false;
  if (d->max_queries < 1 || d->top_k < 1) return false;
  if ((int64_t)d->max_queries * d->top_k > HSK_MAX_SELECTIONS_PER_REQUEST) return false;
  if (d->max_ctx < 1 || d->max_ctx > 0x7fffffffLL || !d->ctx_len) return false;
  if (d->gather_mode != HSK_GATHER_ZEROCOPY && d->gather_mode != HSK_GATHER_NO_IO &&
      d->gather_mode != HSK_GATHER_DEFERRED)
    return false;
  if (d->gather_blocks < 0 || d->host_alias_sources < 0 || d->host_alias_sources > 1) return false;
  for (int32_t r = 0; r < d->num_requests; ++r)
    if (d->ctx_len[r] < 1 || d->ctx_len[r] > d->max_ctx) return false;
  if (d->staging_arenas < 0 || d->staging_arenas > d->num_sources) return false;
  if (total_pool_rows(*d) > 0x7fffffffLL) return false;  // locations are int32 rows
  return true;
}

bool layout_workspace(const hsk_desc& d, WorkspaceLayout* L) {
  const int64_t R = d.num_requests, B = d.hot_slots;
  const int64_t max_pages = d.page_rows ? d.max_ctx / d.page_rows : 0;
  const int64_t cap = (int64_t)d.max_queries * d.top_k;
  int64_t off = 0;
  L->ctx = off; off = align_up(off + 8 * R * d.num_sources);
  L->wt_pos = off; off = align_up(off + 4 * 2 * R * d.num_sources);
  L->err = off; off = align_up(off + 4);
  // fill codes of the fused resolve + attend, which serves stores with one query per request
  L->fill = off; off = align_up(off + (d.max_queries == 1 ? 4 * R * cap : 0));
  L->key.clear(); L->rec.clear(); L->order.clear(); L->pt.clear(); L->opt.clear();
  L->plan_n.clear(); L->plan_pos.clear(); L->plan_dst.clear(); L->ready.clear();
  for (int32_t s = 0; s < d.num_sources; ++s) {
    L->key.push_back(off); off = align_up(off + 4 * R * B);
    L->rec.push_back(off); off = align_up(off + 4 * R * B);
    L->order.push_back(off); off = align_up(off + 2 * R * B);
    L->pt.push_back(off); off = align_up(off + 4 * R * d.max_ctx);
    L->opt.push_back(off); off = align_up(off + 4 * R * max_pages);
    L->plan_n.push_back(off); off = align_up(off + 4 * R);
    L->plan_pos.push_back(off); off = align_up(off + 4 * R * cap);
    L->plan_dst.push_back(off); off = align_up(off + 4 * R * cap);
    L->ready.push_back(off); off = align_up(off + 4 * R);
  }
  L->total = off;
  return true;
}

}  // namespace hsk

using namespace hsk;

extern "C" {

const char* hsk_status_str(hsk_status s) {
  switch (s) {
    case HSK_OK: return "HSK_OK";
    case HSK_EINVAL: return "HSK_EINVAL: bad argument or shape";
    case HSK_ENOMEM: return "HSK_ENOMEM: pinned host allocation failed";
    case HSK_EHIP: return "HSK_EHIP: HIP runtime call failed";
    case HSK_ESTATE: return "HSK_ESTATE: call not valid in this state";
    case HSK_ERANGE: return "HSK_ERANGE: selected position outside the request's history";
    case HSK_ESTAGE: return "HSK_ESTAGE: missing rows exceed free hot slots plus staging";
    case HSK_EEPOCH: return "HSK_EEPOCH: epoch not greater than the source's last epoch";
    case HSK_EWAIT: return "HSK_EWAIT: admission waits, optional pages cannot cover its capacity";
    case HSK_ESCRATCH: return "HSK_ESCRATCH: the call needs more scratch than the static buffer holds";
    default: return "unknown hsk_status";
  }
}

hsk_status hsk_workspace_bytes(const hsk_desc* desc, size_t* workspace_bytes, size_t* pool_bytes) {
  if (!valid_desc(desc) || !workspace_bytes || !pool_bytes) return HSK_EINVAL;
  WorkspaceLayout L;
  layout_workspace(*desc, &L);
  *workspace_bytes = (size_t)L.total;
  *pool_bytes = (size_t)total_pool_rows(*desc) * desc->row_bytes;
  return HSK_OK;
}

void hsk_kv_store_destroy(hsk_store* st) {
  if (!st) return;
  (void)hipDeviceSynchronize();
  residency_destroy(st);
  for (hipEvent_t e : st->wt_done)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : st->tail_done)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : st->fetched)
    if (e) (void)hipEventDestroy(e);
  for (char* h : st->host)
    if (h) (void)hipHostFree(h);
  if (st->h_stage) (void)hipHostFree(st->h_stage);
  delete st;
}

hsk_status hsk_kv_store_init(const hsk_desc* desc, void* d_workspace, void* d_pool, hsk_stream_t stream,
                             hsk_store** out) {
  if (!out) return HSK_EINVAL;
  *out = nullptr;
  if (!valid_desc(desc) || !d_workspace || !d_pool) return HSK_EINVAL;
  if (((uintptr_t)d_workspace % kAlign) || ((uintptr_t)d_pool % kAlign)) return HSK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  hsk_store* st = new (std::nothrow) hsk_store();
  if (!st) return HSK_ENOMEM;
  st->d = *desc;
  st->n_import.assign(desc->ctx_len, desc->ctx_len + desc->num_requests);
  st->d.ctx_len = st->n_import.data();
  const int32_t R = desc->num_requests, B = desc->hot_slots;
  st->ctx.clear();
  for (int32_t k = 0; k < desc->num_sources; ++k) st->ctx.insert(st->ctx.end(), st->n_import.begin(), st->n_import.end());
  st->max_pages = desc->page_rows ? desc->max_ctx / desc->page_rows : 0;
  st->plan_cap = desc->max_queries * desc->top_k;
  st->rows_per_src = rows_per_source(*desc);
  st->host_sources = desc->host_alias_sources ? 1 : desc->num_sources;
  st->ws = (char*)d_workspace;
  st->pool = (char*)d_pool;
  if (hipGetDevice(&st->device) != hipSuccess) { delete st; return HSK_EHIP; }
  WorkspaceLayout L;
  layout_workspace(*desc, &L);
  st->d_ctx = (int64_t*)(st->ws + L.ctx);
  st->d_wt_pos = (int32_t*)(st->ws + L.wt_pos);
  st->wt_done.assign(2 * (size_t)desc->num_sources, nullptr);
  st->wt_pending.assign(2 * (size_t)desc->num_sources, 0);
  st->tail_done.assign((size_t)desc->num_sources, nullptr);
  st->append_parity.assign((size_t)desc->num_sources, 0);
  st->fetched.assign((size_t)desc->num_sources, nullptr);
  // A fetched event orders one stream of this device after a copy kernel on another: device scope is all its
  // release and acquire need (the rows it copied are read by kernels of this device only), and without the
  // system-scope fences the copy stream's next fetch starts ~2 us sooner.  The copy kernel's launch records it
  // (hipExtLaunchKernel's stop event, which takes an event that keeps timing), so no marker follows the kernel.
  for (hipEvent_t& e : st->fetched)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      e = nullptr;
      hsk_kv_store_destroy(st);
      return HSK_EHIP;
    }
  for (hipEvent_t& e : st->wt_done)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) { e = nullptr; hsk_kv_store_destroy(st); return HSK_EHIP; }
  for (hipEvent_t& e : st->tail_done)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) { e = nullptr; hsk_kv_store_destroy(st); return HSK_EHIP; }
  st->d_err = (int32_t*)(st->ws + L.err);
  st->d_fill = (int32_t*)(st->ws + L.fill);
  for (int32_t k = 0; k < desc->num_sources; ++k) {
    SourceMeta m;
    m.key = (int32_t*)(st->ws + L.key[k]);
    m.rec = (uint32_t*)(st->ws + L.rec[k]);
    m.order = (uint16_t*)(st->ws + L.order[k]);
    m.pt = (int32_t*)(st->ws + L.pt[k]);
    m.opt = st->max_pages ? (int32_t*)(st->ws + L.opt[k]) : nullptr;
    m.plan_n = (int32_t*)(st->ws + L.plan_n[k]);
    m.plan_pos = (int32_t*)(st->ws + L.plan_pos[k]);
    m.plan_dst = (int32_t*)(st->ws + L.plan_dst[k]);
    m.ready = (uint32_t*)(st->ws + L.ready[k]);
    st->meta.push_back(m);
  }
  st->last_epoch.assign(desc->num_sources, 0u);
  st->replay_dst.assign(desc->num_sources, 0);
  st->opt_mirror.assign((size_t)desc->num_sources * R, std::vector<int32_t>());
  for (auto& v : st->opt_mirror) v.assign((size_t)st->max_pages, -1);
  // pinned, device-mapped host rows
  const size_t host_bytes = (size_t)R * (size_t)desc->max_ctx * (size_t)desc->row_bytes;
  for (int32_t k = 0; k < st->host_sources; ++k) {
    void* h = nullptr;
    if (hipHostMalloc(&h, host_bytes, hipHostMallocMapped) != hipSuccess || !h) {
      (void)hipGetLastError();
      hsk_kv_store_destroy(st);
      return HSK_ENOMEM;
    }
    st->host.push_back((char*)h);
  }
  st->h_stage_bytes = std::max<size_t>(1 << 20, (size_t)st->max_pages * sizeof(CopyRun) + 4 * (size_t)st->max_pages);
  if (hipHostMalloc(&st->h_stage, st->h_stage_bytes, hipHostMallocMapped) != hipSuccess) {
    (void)hipGetLastError();
    hsk_kv_store_destroy(st);
    return HSK_ENOMEM;
  }
  // metadata: empty caches, slot order 0..B-1
  if (hipMemcpyAsync(st->d_ctx, st->ctx.data(), sizeof(int64_t) * st->ctx.size(), hipMemcpyHostToDevice, s) !=
          hipSuccess ||
      launch_fill_i32(st->d_err, 1, 0, s) != hipSuccess) {
    hsk_kv_store_destroy(st);
    return HSK_EHIP;
  }
  for (int32_t k = 0; k < desc->num_sources; ++k) {
    if (launch_init_meta(st->meta[k], R, B, desc->max_ctx, st->max_pages, s) != hipSuccess) {
      hsk_kv_store_destroy(st);
      return HSK_EHIP;
    }
  }
  // the context-length copy reads pageable host memory owned by the store: wait for it
  if (hipStreamSynchronize(s) != hipSuccess) { hsk_kv_store_destroy(st); return HSK_EHIP; }
  *out = st;
  return HSK_OK;
}

hsk_status hsk_host_rows(hsk_store* st, int32_t source, int32_t req, void** h_rows, int64_t* n_rows) {
  if (!st || !h_rows || !n_rows || source < 0 || source >= st->d.num_sources || req < 0 ||
      req >= st->d.num_requests)
    return HSK_EINVAL;
  const int32_t hs = st->d.host_alias_sources ? 0 : source;
  *h_rows = st->host[hs] + (size_t)req * (size_t)st->d.max_ctx * (size_t)st->d.row_bytes;
  *n_rows = st->d.max_ctx;
  return HSK_OK;
}

hsk_status hsk_pool_base(hsk_store* st, int32_t source, void** d_pool_source) {
  if (!st || !d_pool_source || source < 0 || source >= st->d.num_sources) return HSK_EINVAL;
  *d_pool_source = st->pool + (size_t)source * (size_t)st->rows_per_src * (size_t)st->d.row_bytes;
  return HSK_OK;
}

hsk_status hsk_commit_prefill(hsk_store* st, hsk_stream_t stream) {
  if (!st) return HSK_EINVAL;
  if (st->res) return HSK_ESTATE;  // admissions place the tails
  if (st->d.tail_rows == 0) return HSK_OK;
  const int64_t stride = st->d.max_ctx * (int64_t)st->d.row_bytes;
  for (int32_t k = 0; k < st->d.num_sources; ++k) {
    void* pool;
    hsk_pool_base(st, k, &pool);
    const int32_t hs = st->d.host_alias_sources ? 0 : k;
    HSK_HIP(launch_tail_copy(st->host[hs], stride, (char*)pool, st->d_ctx + (size_t)k * st->d.num_requests,
                             st->d.num_requests, st->d.hot_slots, st->d.tail_rows, st->d.row_bytes,
                             (hipStream_t)stream));
  }
  return HSK_OK;
}

hsk_status hsk_residency_set(hsk_store* st, int32_t source, int32_t req, const int32_t* h_page_ids,
                             int64_t n_pages, hsk_stream_t stream) {
  if (!st || source < 0 || source >= st->d.num_sources || req < 0 || req >= st->d.num_requests) return HSK_EINVAL;
  if (st->d.page_rows == 0 || st->res) return HSK_ESTATE;  // scheduled residency owns the maps
  // only whole pages of the history imported at admission may be held optionally (Adaptive DHiSparse
  // section 3.1); rows produced while decoding are handled by the tail and the hot cache instead
  const int64_t complete = st->n_import[req] / st->d.page_rows;
  if (n_pages < 0 || n_pages > complete || (n_pages > 0 && !h_page_ids)) return HSK_EINVAL;
  for (int64_t g = 0; g < n_pages; ++g)
    if (h_page_ids[g] < -1 || h_page_ids[g] >= st->d.opt_pool_pages) return HSK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t>& mirror = st->opt_mirror[(size_t)source * st->d.num_requests + req];
  const int64_t P = st->d.page_rows, rb = st->d.row_bytes;
  const int64_t opt_base_row = (int64_t)st->d.num_requests * st->d.hot_slots + (int64_t)st->d.num_requests * st->d.tail_rows;
  int32_t* d_map = st->meta[source].opt + (size_t)req * st->max_pages;
  bool all_drop = true, any_change = false;
  for (int64_t g = 0; g < n_pages; ++g) {
    if (h_page_ids[g] >= 0) all_drop = false;
    if (h_page_ids[g] != mirror[g]) any_change = true;
  }
  if (!any_change) return HSK_OK;
  if (all_drop) {
    // reclaim: clear the ready locations in stream order, after earlier readers; no host staging needed
    HSK_HIP(launch_fill_i32(d_map, n_pages, -1, s));
    for (int64_t g = 0; g < n_pages; ++g) mirror[g] = -1;
    return HSK_OK;
  }
  // population: copy newly mapped pages, then publish the map after the copies (same stream)
  CopyRun* runs = (CopyRun*)st->h_stage;
  int32_t* map_stage = (int32_t*)((char*)st->h_stage + sizeof(CopyRun) * (size_t)st->max_pages);
  int32_t nrun = 0;
  const int64_t host_off = (int64_t)req * st->d.max_ctx * rb;
  for (int64_t g = 0; g < n_pages; ++g) {
    int32_t id = h_page_ids[g];
    if (id < 0 || id == mirror[g]) continue;
    int64_t src = host_off + g * P * rb;
    int64_t dst = (opt_base_row + (int64_t)id * P) * rb;
    if (nrun > 0 && runs[nrun - 1].src + runs[nrun - 1].bytes == src && runs[nrun - 1].dst + runs[nrun - 1].bytes == dst) {
      runs[nrun - 1].bytes += P * rb;
    } else {
      runs[nrun].src = src; runs[nrun].dst = dst; runs[nrun].bytes = P * rb;
      ++nrun;
    }
  }
  for (int64_t g = 0; g < n_pages; ++g) map_stage[g] = h_page_ids[g];
  void* pool;
  hsk_pool_base(st, source, &pool);
  const int32_t hs = st->d.host_alias_sources ? 0 : source;
  if (nrun > 0) HSK_HIP(launch_copy_runs(st->host[hs], (char*)pool, runs, nrun, s));
  HSK_HIP(hipMemcpyAsync(d_map, map_stage, sizeof(int32_t) * (size_t)n_pages, hipMemcpyHostToDevice, s));
  HSK_HIP(hipStreamSynchronize(s));  // the staging buffer is reused by the next call
  for (int64_t g = 0; g < n_pages; ++g) mirror[g] = h_page_ids[g];
  return HSK_OK;
}

hsk_status hsk_reclaim_plan(const int64_t* h_pages_held, int32_t n, int64_t deficit, int32_t* q_out) {
  if (!q_out || n < 0 || (n > 0 && !h_pages_held)) return HSK_EINVAL;
  if (deficit <= 0) { *q_out = 0; return HSK_OK; }
  int64_t acc = 0;
  for (int32_t q = 0; q < n; ++q) {
    if (h_pages_held[q] < 0) return HSK_EINVAL;
    acc += h_pages_held[q];
    if (acc >= deficit) { *q_out = q + 1; return HSK_OK; }
  }
  *q_out = -1;
  return HSK_OK;
}

static int32_t gather_blocks_for(const hsk_store* st) {
  if (st->d.gather_blocks > 0) return st->d.gather_blocks;
  return 32;  // 512 waves: rows are spread evenly over them whatever the batch (the host link fills from ~256)
}

static ResolveArgs resolve_args(hsk_store* st, int32_t source, uint32_t epoch, const int32_t* d_sel,
                                const int32_t* d_nq, int32_t* d_locs, hsk_stats* d_stats) {
  ResolveArgs a;
  a.sel = d_sel; a.nq = d_nq; a.locs = d_locs; a.stats = d_stats;
  a.ctx = st->d_ctx + (size_t)source * st->d.num_requests; a.m = st->meta[source];
  a.err = st->d_err; a.fill = nullptr; a.max_ctx = st->d.max_ctx; a.max_pages = st->max_pages;
  a.host = nullptr; a.pool = nullptr; a.host_req_stride = 0; a.ready = nullptr;
  const int64_t R = st->d.num_requests;
  a.opt_base = R * st->d.hot_slots + R * st->d.tail_rows;
  a.stg_base = stg_base_of(st->d, source);
  a.plan_cap = st->plan_cap;
  a.R = st->d.num_requests; a.B = st->d.hot_slots; a.T = st->d.tail_rows; a.P = st->d.page_rows;
  a.S = st->d.staging_rows; a.Qmax = st->d.max_queries; a.k = st->d.top_k; a.row_bytes = st->d.row_bytes;
  a.epoch = epoch;
  return a;
}

hsk_status hsk_resolve_step(hsk_store* st, int32_t source, uint32_t epoch, const int32_t* d_sel, const int32_t* d_nq,
                            int32_t* d_locs, hsk_stats* d_stats, hsk_stream_t stream) {
  if (!st || source < 0 || source >= st->d.num_sources || !d_sel || !d_locs) return HSK_EINVAL;
  if (st->replay_dst[source]) return HSK_ESTATE;  // its pool rows follow another source's slot table
  if (epoch <= st->last_epoch[source] || epoch > 0x7fffffffu) return HSK_EEPOCH;
  hipStream_t s = (hipStream_t)stream;
  ResolveArgs a = resolve_args(st, source, epoch, d_sel, d_nq, d_locs, d_stats);
  if (st->d.gather_mode == HSK_GATHER_ZEROCOPY) {
    // the resolving workgroups copy their requests' missing rows themselves (zero-copy host reads)
    void* pool;
    hsk_pool_base(st, source, &pool);
    const int32_t hs = st->d.host_alias_sources ? 0 : source;
    a.host = st->host[hs];
    a.pool = (char*)pool;
    a.host_req_stride = st->d.max_ctx * (int64_t)st->d.row_bytes;
  }
  HSK_HIP(launch_resolve(a, s));
  st->last_epoch[source] = epoch;
  return HSK_OK;
}

hsk_status hsk_resolve_attend(hsk_store* st, int32_t source, uint32_t epoch, const int32_t* d_sel, int32_t* d_locs,
                              hsk_stats* d_stats, const hsk_attn_desc* desc, const void* d_q, void* d_out,
                              void* d_scratch, size_t scratch_bytes, hsk_stream_t stream) {
  if (!st || source < 0 || source >= st->d.num_sources || !d_sel || !d_locs || !desc || !d_q || !d_out ||
      !d_scratch)
    return HSK_EINVAL;
  // one query per request, host rows copied on the device, positions that fit the fill codes, and an
  // attention shape that reads this store's rows, whole (the kernel writes back the dk columns it loads)
  if (st->d.gather_mode != HSK_GATHER_ZEROCOPY || st->d.max_queries != 1 || st->d.max_ctx >= (1 << 30) ||
      desc->kind != HSK_ATTN_MLA || desc->num_requests != st->d.num_requests || desc->max_queries != 1 ||
      desc->top_k != st->d.top_k || (int64_t)desc->row_elems * 2 != st->d.row_bytes || desc->row_elems != desc->dk)
    return HSK_EINVAL;
  if (st->replay_dst[source]) return HSK_ESTATE;
  if (epoch <= st->last_epoch[source] || epoch > 0x7fffffffu) return HSK_EEPOCH;
  hipStream_t s = (hipStream_t)stream;
  ResolveArgs a = resolve_args(st, source, epoch, d_sel, nullptr, d_locs, d_stats);
  a.fill = st->d_fill;
  void* pool;
  hsk_pool_base(st, source, &pool);
  const int32_t hs = st->d.host_alias_sources ? 0 : source;
  // the attention shape is checked before anything is queued, so a rejected call leaves the store as it was
  if (check_mla_fused(desc, d_scratch, scratch_bytes) != HSK_OK) return HSK_EINVAL;
  HSK_HIP(launch_resolve(a, s));
  st->last_epoch[source] = epoch;
  return launch_mla_fused(desc, d_q, (const char*)pool, d_locs, st->d_fill, st->host[hs],
                          st->d.max_ctx * (int64_t)st->d.row_bytes, d_out, d_scratch, scratch_bytes, s);
}

// ready: wait inside the copy kernel for each request's plan of resolve `epoch` (published by a resolve on
// another stream); null: the plan is complete when the kernel starts (stream order)
static hsk_status gather_plan(hsk_store* st, int32_t plan_source, int32_t dst_source, hipStream_t s,
                              const uint32_t* ready = nullptr, uint32_t epoch = 0, hipEvent_t done = nullptr) {
  void* pool;
  hsk_pool_base(st, dst_source, &pool);
  GatherArgs g;
  const int32_t hs = st->d.host_alias_sources ? 0 : dst_source;
  g.host = st->host[hs]; g.pool = (char*)pool;
  g.plan_n = st->meta[plan_source].plan_n; g.plan_pos = st->meta[plan_source].plan_pos;
  g.plan_dst = st->meta[plan_source].plan_dst;
  g.host_req_stride = st->d.max_ctx * (int64_t)st->d.row_bytes;
  g.plan_cap = st->plan_cap; g.row_bytes = st->d.row_bytes;
  g.ready = ready; g.err = st->d_err; g.epoch = epoch;
  HSK_HIP(launch_gather(g, st->d.num_requests, gather_blocks_for(st), s, done));
  return HSK_OK;
}

hsk_status hsk_stream_create(hsk_stream_t* stream) {
  if (!stream) return HSK_EINVAL;
  *stream = nullptr;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    return HSK_EHIP;
  std::vector<uint32_t> mask((size_t)(ncu + 31) / 32, 0xFFFFFFFFu);
  hipStream_t s = nullptr;
  if (hipExtStreamCreateWithCUMask(&s, (uint32_t)mask.size(), mask.data()) != hipSuccess || !s) {
    (void)hipGetLastError();
    return HSK_EHIP;
  }
  *stream = (hsk_stream_t)s;
  return HSK_OK;
}

hsk_status hsk_stream_destroy(hsk_stream_t stream) {
  if (!stream) return HSK_EINVAL;
  return hipStreamDestroy((hipStream_t)stream) == hipSuccess ? HSK_OK : HSK_EHIP;
}

hsk_status hsk_resolve_fetch_attend(hsk_store* st, int32_t source, uint32_t epoch, const int32_t* d_sel,
                                    const int32_t* d_nq, int32_t* d_locs, hsk_stats* d_stats, const hsk_attn_desc* desc,
                                    const void* d_q, void* d_out, void* d_scratch, size_t scratch_bytes,
                                    hsk_stream_t stream, hsk_stream_t copy_stream) {
  if (!st || source < 0 || source >= st->d.num_sources || !d_sel || !d_locs || !desc || !d_q || !d_out ||
      !d_scratch)
    return HSK_EINVAL;
  if (st->d.gather_mode != HSK_GATHER_DEFERRED) return HSK_EINVAL;
  // the attention reads this store's rows at the emitted locations: the same resolution units (requests, or
  // request x KV head for GQA pages), queries, k and row width
  const int64_t units = desc->kind == HSK_ATTN_GQA ? (int64_t)desc->num_requests * desc->kv_heads : desc->num_requests;
  if (units != st->d.num_requests || desc->max_queries != st->d.max_queries || desc->top_k != st->d.top_k ||
      (int64_t)desc->row_elems * 2 != st->d.row_bytes)
    return HSK_EINVAL;
  size_t need = 0;
  if (hsk_attn_scratch_bytes(desc, &need) != HSK_OK || scratch_bytes < need || ((uintptr_t)d_scratch % 256))
    return HSK_EINVAL;
  if (st->replay_dst[source]) return HSK_ESTATE;
  if (epoch <= st->last_epoch[source] || epoch > 0x7fffffffu) return HSK_EEPOCH;
  hipStream_t s = (hipStream_t)stream, c = (hipStream_t)copy_stream;
  ResolveArgs a = resolve_args(st, source, epoch, d_sel, d_nq, d_locs, d_stats);
  // On two streams the copy does not wait for the resolve through the streams: each resolve workgroup
  // publishes its request's plan with the call's epoch and the copy kernel waits for it, so consecutive
  // copies on the copy stream follow each other without a cross-stream wait in between.
  if (c != s) a.ready = st->meta[source].ready;
  HSK_HIP(launch_resolve(a, s));
  st->last_epoch[source] = epoch;
  // on two streams the copy kernel's launch records the fetched event that the attention's stream waits for
  const hsk_status f = c != s ? gather_plan(st, source, source, c, st->meta[source].ready, epoch, st->fetched[source])
                              : gather_plan(st, source, source, c);
  if (f != HSK_OK) return f;
  if (c != s) HSK_HIP(hipStreamWaitEvent(s, st->fetched[source], 0));
  void* pool;
  hsk_pool_base(st, source, &pool);
  return hsk_sparse_decode_attn(desc, d_q, pool, d_locs, d_nq, d_out, d_scratch, scratch_bytes, stream);
}

hsk_status hsk_append_rows(hsk_store* st, int32_t source, const void* d_rows, int32_t count, hsk_stream_t stream,
                           hsk_stream_t backup_stream) {
  if (!st || source < 0 || source >= st->d.num_sources || !d_rows || count < 1 || 2 * count > st->d.tail_rows ||
      st->d.host_alias_sources)
    return HSK_EINVAL;
  const int32_t R = st->d.num_requests;
  int64_t* hctx = st->ctx.data() + (size_t)source * R;
  for (int32_t r = 0; r < R; ++r)  // free slots (context -1) are skipped
    if (hctx[r] >= 0 && hctx[r] + count > st->d.max_ctx) return HSK_EINVAL;
  hipStream_t s = (hipStream_t)stream, b = (hipStream_t)backup_stream;
  const int par = st->append_parity[source];
  const size_t ev = 2 * (size_t)source + par;
  void* pool;
  hsk_pool_base(st, source, &pool);
  int32_t* wt_pos = st->d_wt_pos + ((size_t)source * 2 + par) * R;
  // The write-through of the append before last (same parity) reads tail rows that this append may overwrite,
  // and its rows can leave the tail from this append on: the stream waits for it.  The last append's rows stay
  // in the tail (2 count <= T), so its write-through keeps running beside the stream.
  if (st->wt_pending[ev]) {
    HSK_HIP(hipStreamWaitEvent(s, st->wt_done[ev], 0));
    st->wt_pending[ev] = 0;
  }
  HSK_HIP(launch_append_tail((const char*)d_rows, (char*)pool, st->d_ctx + (size_t)source * R, wt_pos, R,
                             st->d.hot_slots, st->d.tail_rows, count, st->d.row_bytes, s));
  if (b != s) {
    HSK_HIP(hipEventRecord(st->tail_done[source], s));
    HSK_HIP(hipStreamWaitEvent(b, st->tail_done[source], 0));
  }
  HSK_HIP(launch_write_through((const char*)pool, st->host[source], st->d.max_ctx * (int64_t)st->d.row_bytes, wt_pos,
                               R, st->d.hot_slots, st->d.tail_rows, count, st->d.row_bytes, b));
  HSK_HIP(hipEventRecord(st->wt_done[ev], b));
  st->wt_pending[ev] = 1;
  st->append_parity[source] = par ^ 1;
  for (int32_t r = 0; r < R; ++r)
    if (hctx[r] >= 0) hctx[r] += count;
  return HSK_OK;
}

hsk_status hsk_completed_rows(int64_t n_before, int64_t n_after, int32_t m, int64_t* first, int64_t* count) {
  if (!first || !count || m < 1 || n_before < 0 || n_after < n_before) return HSK_EINVAL;
  *first = n_before / m;
  *count = n_after / m - n_before / m;
  return HSK_OK;
}

hsk_status hsk_ring_rows(int64_t window, int32_t page_rows, int32_t k_max, int64_t* ring_rows) {
  if (!ring_rows || window < 1 || page_rows < 1 || k_max < 1) return HSK_EINVAL;
  const int64_t need = window + page_rows - 1 + k_max;     // Eq. 9
  *ring_rows = (need + page_rows - 1) / page_rows * page_rows;
  return HSK_OK;
}

hsk_status hsk_ring_write(void* d_ring, int64_t ring_rows, int32_t slots, const void* d_rows, int32_t count,
                          int32_t row_bytes, const int64_t* d_t0, hsk_stream_t stream) {
  if (!d_ring || !d_rows || !d_t0 || slots < 1 || count < 1 || ring_rows < count || row_bytes < 16 ||
      row_bytes % 16)
    return HSK_EINVAL;
  HSK_HIP(launch_ring_write((char*)d_ring, ring_rows, slots, (const char*)d_rows, count, row_bytes, d_t0,
                            (hipStream_t)stream));
  return HSK_OK;
}

hsk_status hsk_ring_window_locs(int64_t ring_rows, int32_t slots, int32_t window, const int64_t* d_t_end,
                                int32_t* d_locs, hsk_stream_t stream) {
  if (!d_t_end || !d_locs || slots < 1 || window < 1 || window > ring_rows || (int64_t)slots * ring_rows > 0x7fffffffLL)
    return HSK_EINVAL;
  HSK_HIP(launch_ring_locs(ring_rows, slots, window, d_t_end, d_locs, (hipStream_t)stream));
  return HSK_OK;
}

hsk_status hsk_context_rows(hsk_store* st, int32_t source, int32_t req, int64_t* n_rows) {
  if (!st || !n_rows || source < 0 || source >= st->d.num_sources || req < 0 || req >= st->d.num_requests)
    return HSK_EINVAL;
  *n_rows = st->ctx[(size_t)source * st->d.num_requests + req];
  return HSK_OK;
}

// The rows of plan_source's last miss plan, from dst_source's host rows into dst_source's pool at the plan's
// pool rows: the gather kernel, gather_blocks workgroups.
hsk_status hsk_replay_plan(hsk_store* st, int32_t plan_source, int32_t dst_source, hsk_stream_t stream) {
  if (!st || plan_source < 0 || plan_source >= st->d.num_sources || dst_source < 0 ||
      dst_source >= st->d.num_sources || plan_source == dst_source)
    return HSK_EINVAL;
  if (st->d.staging_arenas && st->d.staging_rows) return HSK_EINVAL;
  // A destination's pool rows follow the plan source's slot table, not its own metadata: it never resolves
  // again (HSK_ESTATE), and it cannot serve as a plan source, having no plan of its own.
  if (st->replay_dst[plan_source] || st->last_epoch[dst_source] != 0) return HSK_ESTATE;
  st->replay_dst[dst_source] = 1;
  if (st->d.gather_mode == HSK_GATHER_NO_IO) return HSK_OK;
  return gather_plan(st, plan_source, dst_source, (hipStream_t)stream);
}

hsk_status hsk_fetch_plan(hsk_store* st, int32_t source, hsk_stream_t stream) {
  if (!st || source < 0 || source >= st->d.num_sources || st->d.gather_mode != HSK_GATHER_DEFERRED)
    return HSK_EINVAL;
  if (st->last_epoch[source] == 0 || st->replay_dst[source]) return HSK_ESTATE;
  return gather_plan(st, source, source, (hipStream_t)stream);
}

hsk_status hsk_promote_staged(hsk_store* st, int32_t source, const int32_t* d_locs, const int32_t* d_nq,
                              const int32_t* d_accepted, int32_t* d_promoted, hsk_stream_t stream) {
  if (!st || source < 0 || source >= st->d.num_sources || !d_locs || !d_accepted) return HSK_EINVAL;
  if (st->last_epoch[source] == 0 || st->replay_dst[source]) return HSK_ESTATE;
  if (st->d.staging_rows > HSK_MAX_SELECTIONS_PER_REQUEST) return HSK_EINVAL;  // the kernel's staging bitmap
  hipStream_t s = (hipStream_t)stream;
  if (st->d.staging_rows == 0) {  // nothing can be staged: nothing to promote
    if (d_promoted) HSK_HIP(launch_fill_i32(d_promoted, st->d.num_requests, 0, s));
    return HSK_OK;
  }
  void* pool;
  hsk_pool_base(st, source, &pool);
  HSK_HIP(launch_promote(d_locs, d_nq, d_accepted, d_promoted, st->meta[source], (char*)pool, st->d.max_ctx,
                         stg_base_of(st->d, source), st->d.num_requests, st->d.hot_slots, st->d.staging_rows,
                         st->d.max_queries, st->d.top_k, st->d.row_bytes, st->last_epoch[source], s));
  return HSK_OK;
}

hsk_status hsk_snapshot(hsk_store* st, int32_t source, int32_t req, int32_t* key, uint32_t* rec, uint16_t* order,
                        int32_t* pt, int32_t* opt) {
  if (!st || source < 0 || source >= st->d.num_sources || req < 0 || req >= st->d.num_requests) return HSK_EINVAL;
  HSK_HIP(hipDeviceSynchronize());
  const SourceMeta& m = st->meta[source];
  const size_t B = st->d.hot_slots;
  if (key) HSK_HIP(hipMemcpy(key, m.key + req * B, 4 * B, hipMemcpyDeviceToHost));
  if (rec) HSK_HIP(hipMemcpy(rec, m.rec + req * B, 4 * B, hipMemcpyDeviceToHost));
  if (order) HSK_HIP(hipMemcpy(order, m.order + req * B, 2 * B, hipMemcpyDeviceToHost));
  const size_t n_r = (size_t)std::max<int64_t>(0, st->ctx[(size_t)source * st->d.num_requests + req]);
  if (pt) HSK_HIP(hipMemcpy(pt, m.pt + (size_t)req * st->d.max_ctx, 4 * n_r, hipMemcpyDeviceToHost));
  if (opt && st->max_pages) {
    const size_t np = (size_t)(st->n_import[req] / st->d.page_rows);
    if (np) HSK_HIP(hipMemcpy(opt, m.opt + (size_t)req * st->max_pages, 4 * np, hipMemcpyDeviceToHost));
  }
  return HSK_OK;
}

hsk_status hsk_read_plan(hsk_store* st, int32_t source, int32_t req, int32_t* pos, int32_t* dst, int32_t cap,
                         int32_t* n) {
  if (!st || !n || source < 0 || source >= st->d.num_sources || req < 0 || req >= st->d.num_requests || cap < 0)
    return HSK_EINVAL;
  HSK_HIP(hipDeviceSynchronize());
  const SourceMeta& m = st->meta[source];
  int32_t cnt = 0;
  HSK_HIP(hipMemcpy(&cnt, m.plan_n + req, 4, hipMemcpyDeviceToHost));
  *n = cnt;
  const size_t w = (size_t)std::min(cnt, cap);
  if (w && pos) HSK_HIP(hipMemcpy(pos, m.plan_pos + (size_t)req * st->plan_cap, 4 * w, hipMemcpyDeviceToHost));
  if (w && dst) HSK_HIP(hipMemcpy(dst, m.plan_dst + (size_t)req * st->plan_cap, 4 * w, hipMemcpyDeviceToHost));
  return HSK_OK;
}

hsk_status hsk_sync_status(hsk_store* st, hsk_stream_t stream) {
  if (!st) return HSK_EINVAL;
  HSK_HIP(hipStreamSynchronize((hipStream_t)stream));
  int32_t e = 0;
  HSK_HIP(hipMemcpy(&e, st->d_err, 4, hipMemcpyDeviceToHost));
  if (e != 0) {
    HSK_HIP(launch_fill_i32(st->d_err, 1, 0, (hipStream_t)stream));
    HSK_HIP(hipStreamSynchronize((hipStream_t)stream));
  }
  return e;
}

}  // extern "C"
