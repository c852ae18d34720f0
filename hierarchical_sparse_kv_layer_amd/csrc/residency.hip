// Load-adaptive residency ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy",
// section 3.1, Eqs. 3-4): admission of requests into slots, optional residency of their imported history
// under a capacity bound, reclaim of whole requests with backup before retire, and bounded round-robin
// repopulation whose ready locations are published only after their copies complete.
//
// The scheduler is host code: it decides which pages move and queues the moves.  The moves are three small
// kernels: a chunked copy (host <-> pool, device -> pool), a scatter of optional-map entries over every
// source, and a per-slot metadata reset.  Copy and map lists are staged in a ring of pinned, device-mapped
// buffers, each guarded by an event recorded after the kernel that reads it.
#include <algorithm>
#include <deque>
#include <functional>
#include <queue>
#include <vector>

#include "hsk_internal.h"

namespace hsk {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int64_t kChunkBytes = 64 << 10;   // one workgroup per <= 64 KiB piece of a run
constexpr int kStageSlots = 4;
constexpr size_t kStageBytes = 1 << 20;
constexpr uint8_t kReady = HSK_PAGE_READY, kBacked = HSK_PAGE_BACKED;

struct MapEntry {
  int32_t idx;   // r * max_pages + g
  int32_t val;   // page id, or -1
};

// ------------------------------------------------------------------------------------------------ kernels
// Each workgroup copies one run piece (<= 64 KiB, 16-byte multiple); four 16-byte loads per lane are in
// flight before their stores, which keeps host-link reads deep enough to stream.
__global__ __launch_bounds__(kCopyThreads) void copy_pieces_kernel(const char* src, char* dst, const CopyRun* runs) {
  const CopyRun run = runs[blockIdx.x];
  const v4u* s = (const v4u*)(src + run.src);
  v4u* d = (v4u*)(dst + run.dst);
  const int64_t n = run.bytes >> 4;
  for (int64_t i = threadIdx.x; i < n; i += 4 * kCopyThreads) {
    v4u v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j * kCopyThreads < n) v[j] = s[i + j * kCopyThreads];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i + j * kCopyThreads < n) d[i + j * kCopyThreads] = v[j];
  }
}

// Optional-map entries of every source (blockIdx.y = source; the sources' maps are meta_stride bytes apart).
__global__ void map_scatter_kernel(char* opt0, int64_t meta_stride, const MapEntry* e, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const MapEntry m = e[i];
  ((int32_t*)(opt0 + (int64_t)blockIdx.y * meta_stride))[m.idx] = m.val;
}

// Slot r of every source (blockIdx.y): empty hot cache (keys -1, recency 0, slot order 0..B-1), page table
// and optional map -1, empty miss plan, context n_rows (-1: free slot).
__global__ void reset_slot_kernel(SourceMeta m, int64_t meta_stride, int64_t* ctx, int32_t r, int32_t R, int32_t B,
                                  int64_t max_ctx, int64_t max_pages, int64_t n_rows) {
  const int64_t off = (int64_t)blockIdx.y * meta_stride;
  int32_t* key = (int32_t*)((char*)m.key + off) + (int64_t)r * B;
  uint32_t* rec = (uint32_t*)((char*)m.rec + off) + (int64_t)r * B;
  uint16_t* order = (uint16_t*)((char*)m.order + off) + (int64_t)r * B;
  int32_t* pt = (int32_t*)((char*)m.pt + off) + (int64_t)r * max_ctx;
  int32_t* opt = m.opt ? (int32_t*)((char*)m.opt + off) + (int64_t)r * max_pages : nullptr;
  const int64_t n = max_ctx > B ? max_ctx : (int64_t)B;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < max_ctx) pt[i] = -1;
    if (i < B) { key[i] = -1; rec[i] = 0u; order[i] = (uint16_t)i; }
    if (opt && i < max_pages) opt[i] = -1;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ((int32_t*)((char*)m.plan_n + off))[r] = 0;
    ctx[(int64_t)blockIdx.y * R + r] = n_rows;
  }
}

__global__ void fill_i64_kernel(int64_t* p, int64_t n, int64_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ------------------------------------------------------------------------------------------------ host state
struct ResidencyState {
  hsk_residency_desc cfg{};
  int64_t meta_stride = 0;
  std::vector<uint8_t> admitted;
  std::vector<int64_t> seq;              // admission order (reclaim order); 0 = free
  int64_t next_seq = 1;
  std::vector<std::vector<int32_t>> ids; // [slot][page] page id or -1
  std::vector<std::vector<uint8_t>> flags;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_ids;
  int32_t cursor = 0;
  int32_t n_admitted = 0;
  int64_t held = 0;
  struct Pending { int32_t r, g, id; int64_t seq; };
  struct Batch { hipEvent_t ev; std::vector<Pending> pages; };
  std::deque<Batch> batches;             // population copies in issue order
  std::vector<hipEvent_t> spare;         // recycled batch events
  hipEvent_t order_ev = nullptr;         // last admission / release / reclaim on the store's stream
  bool order_recorded = false;
  char* stage[kStageSlots] = {};
  hipEvent_t stage_ev[kStageSlots] = {};
  bool stage_busy[kStageSlots] = {};
  int stage_next = 0;
};

void residency_destroy(hsk_store* st) {
  ResidencyState* rs = st->res;
  if (!rs) return;
  for (auto& b : rs->batches) (void)hipEventDestroy(b.ev);
  for (hipEvent_t e : rs->spare) (void)hipEventDestroy(e);
  if (rs->order_ev) (void)hipEventDestroy(rs->order_ev);
  for (int i = 0; i < kStageSlots; ++i) {
    if (rs->stage[i]) (void)hipHostFree(rs->stage[i]);
    if (rs->stage_ev[i]) (void)hipEventDestroy(rs->stage_ev[i]);
  }
  delete rs;
  st->res = nullptr;
}

// A pinned staging buffer whose previous reader has finished; each holder releases its own slot after
// queueing the kernel that reads it.
static hsk_status acquire_stage(ResidencyState* rs, char** out, int* slot) {
  const int i = rs->stage_next;
  rs->stage_next = (i + 1) % kStageSlots;
  if (rs->stage_busy[i]) HSK_HIP(hipEventSynchronize(rs->stage_ev[i]));
  rs->stage_busy[i] = false;
  *out = rs->stage[i];
  *slot = i;
  return HSK_OK;
}

static hsk_status release_stage(ResidencyState* rs, int slot, hipStream_t s) {
  HSK_HIP(hipEventRecord(rs->stage_ev[slot], s));
  rs->stage_busy[slot] = true;
  return HSK_OK;
}

// Byte runs from one base to another, cut into <= 64 KiB pieces, launched when a staging buffer fills.
// Every run is checked against the extent of its source and destination before anything is queued.
class Copier {
 public:
  Copier(ResidencyState* rs, hipStream_t s, const char* src, int64_t src_bytes, char* dst, int64_t dst_bytes)
      : rs_(rs), s_(s), src_(src), dst_(dst), src_bytes_(src_bytes), dst_bytes_(dst_bytes) {}
  hsk_status add(int64_t so, int64_t dof, int64_t bytes) {
    if (so < 0 || dof < 0 || bytes < 0 || so + bytes > src_bytes_ || dof + bytes > dst_bytes_ || (so | dof | bytes) & 15)
      return HSK_EINVAL;
    while (bytes > 0) {
      if (!runs_) {
        if (acquire_stage(rs_, (char**)&runs_, &slot_) != HSK_OK) return HSK_EHIP;
        n_ = 0;
      }
      if (n_ > 0) {
        CopyRun& l = runs_[n_ - 1];
        if (l.src + l.bytes == so && l.dst + l.bytes == dof && l.bytes < kChunkBytes) {
          const int64_t t = std::min(bytes, kChunkBytes - l.bytes);
          l.bytes += t; so += t; dof += t; bytes -= t;
          continue;
        }
      }
      if (n_ == kCap) {
        hsk_status e = flush();
        if (e != HSK_OK) return e;
        continue;
      }
      const int64_t t = std::min(bytes, kChunkBytes);
      runs_[n_++] = CopyRun{so, dof, t};
      so += t; dof += t; bytes -= t;
    }
    return HSK_OK;
  }
  hsk_status flush() {
    if (!runs_) return HSK_OK;
    if (n_ > 0) {
      hipLaunchKernelGGL(copy_pieces_kernel, dim3(n_), dim3(kCopyThreads), 0, s_, src_, dst_, runs_);
      HSK_HIP(hipGetLastError());
    }
    runs_ = nullptr;
    return release_stage(rs_, slot_, s_);
  }

 private:
  static constexpr int32_t kCap = (int32_t)(kStageBytes / sizeof(CopyRun));
  ResidencyState* rs_;
  hipStream_t s_;
  const char* src_;
  char* dst_;
  int64_t src_bytes_, dst_bytes_;
  CopyRun* runs_ = nullptr;
  int32_t n_ = 0;
  int slot_ = 0;
};

// Optional-map entries written to every source's map on one stream.
class MapWriter {
 public:
  MapWriter(hsk_store* st, hipStream_t s) : st_(st), s_(s) {}
  hsk_status add(int32_t r, int32_t g, int32_t val) {
    if (!e_) {
      if (acquire_stage(st_->res, (char**)&e_, &slot_) != HSK_OK) return HSK_EHIP;
      n_ = 0;
    }
    if (r < 0 || r >= st_->d.num_requests || g < 0 || g >= st_->max_pages) return HSK_EINVAL;
    e_[n_++] = MapEntry{(int32_t)(r * st_->max_pages + g), val};
    if (n_ == kCap) return flush();
    return HSK_OK;
  }
  hsk_status flush() {
    if (!e_) return HSK_OK;
    if (n_ > 0) {
      hipLaunchKernelGGL(map_scatter_kernel, dim3((n_ + 255) / 256, st_->d.num_sources), dim3(256), 0, s_,
                         (char*)st_->meta[0].opt, st_->res->meta_stride, e_, n_);
      HSK_HIP(hipGetLastError());
    }
    e_ = nullptr;
    return release_stage(st_->res, slot_, s_);
  }

 private:
  static constexpr int32_t kCap = (int32_t)(kStageBytes / sizeof(MapEntry));
  hsk_store* st_;
  hipStream_t s_;
  MapEntry* e_ = nullptr;
  int32_t n_ = 0;
  int slot_ = 0;
};

static int32_t host_source(const hsk_store* st, int32_t s) { return st->d.host_alias_sources ? 0 : s; }
static char* pool_of(hsk_store* st, int32_t s) {
  return st->pool + (size_t)s * (size_t)st->rows_per_src * (size_t)st->d.row_bytes;
}
static int64_t opt_row0(const hsk_store* st) {
  return (int64_t)st->d.num_requests * st->d.hot_slots + (int64_t)st->d.num_requests * st->d.tail_rows;
}
static int64_t host_req_off(const hsk_store* st, int32_t r) { return (int64_t)r * st->d.max_ctx * st->d.row_bytes; }
static int64_t pool_bytes(const hsk_store* st) { return st->rows_per_src * st->d.row_bytes; }
static int64_t host_bytes(const hsk_store* st) {
  return (int64_t)st->d.num_requests * st->d.max_ctx * st->d.row_bytes;
}

static int64_t free_capacity(const hsk_store* st) {
  const ResidencyState* rs = st->res;
  return rs->cfg.capacity_pages - rs->cfg.reserve_pages - rs->cfg.required_pages * rs->n_admitted - rs->held;
}

static hsk_status reset_slot(hsk_store* st, int32_t r, int64_t n_rows, hipStream_t s) {
  const int64_t n = std::max<int64_t>(st->d.max_ctx, st->d.hot_slots);
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 512);
  hipLaunchKernelGGL(reset_slot_kernel, dim3(blocks, st->d.num_sources), dim3(256), 0, s, st->meta[0],
                     st->res->meta_stride, st->d_ctx, r, st->d.num_requests, st->d.hot_slots, st->d.max_ctx,
                     st->max_pages, n_rows);
  HSK_HIP(hipGetLastError());
  for (int32_t k = 0; k < st->d.num_sources; ++k) st->ctx[(size_t)k * st->d.num_requests + r] = n_rows;
  return HSK_OK;
}

// the stream waits for every population batch that still copies into a page of slot r
static hsk_status wait_pending_of(hsk_store* st, int32_t r, hipStream_t s) {
  for (auto& b : st->res->batches)
    for (const auto& p : b.pages)
      if (p.r == r && p.seq == st->res->seq[r]) {
        HSK_HIP(hipStreamWaitEvent(s, b.ev, 0));
        break;
      }
  return HSK_OK;
}

// the stream waits for write-throughs of earlier appends (they write host rows of every slot)
static hsk_status wait_write_through(hsk_store* st, hipStream_t s) {
  for (size_t i = 0; i < st->wt_done.size(); ++i)
    if (st->wt_pending[i]) HSK_HIP(hipStreamWaitEvent(s, st->wt_done[i], 0));
  return HSK_OK;
}

static hsk_status record_order(hsk_store* st, hipStream_t s) {
  HSK_HIP(hipEventRecord(st->res->order_ev, s));
  st->res->order_recorded = true;
  return HSK_OK;
}

// Eq. 4 in admission order; backup of device-only pages, then retire, all on s.
static hsk_status reclaim_impl(hsk_store* st, int64_t deficit, hipStream_t s, int32_t* out, int32_t* n_out) {
  ResidencyState* rs = st->res;
  if (n_out) *n_out = 0;
  if (deficit <= 0) return HSK_OK;
  std::vector<int32_t> order;
  for (int32_t r = 0; r < st->d.num_requests; ++r)
    if (rs->admitted[r]) order.push_back(r);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return rs->seq[a] < rs->seq[b]; });
  std::vector<int64_t> held(order.size());
  for (size_t i = 0; i < order.size(); ++i)
    for (int32_t id : rs->ids[order[i]]) held[i] += id >= 0;
  int32_t q = -1;
  if (hsk_reclaim_plan(held.data(), (int32_t)held.size(), deficit, &q) != HSK_OK) return HSK_EINVAL;
  if (q < 0) return HSK_EWAIT;
  const int64_t P = st->d.page_rows, rb = st->d.row_bytes, page_bytes = P * rb;
  for (int32_t i = 0; i < q; ++i)
    if (wait_pending_of(st, order[i], s) != HSK_OK) return HSK_EHIP;
  // backup first: pages whose rows exist only on the device are copied to their host rows
  for (int32_t hs = 0; hs < st->host_sources; ++hs) {
    Copier c(rs, s, pool_of(st, hs), pool_bytes(st), st->host[hs], host_bytes(st));
    for (int32_t i = 0; i < q; ++i) {
      const int32_t r = order[i];
      for (size_t g = 0; g < rs->ids[r].size(); ++g)
        if (rs->ids[r][g] >= 0 && !(rs->flags[r][g] & kBacked)) {
          hsk_status e = c.add((opt_row0(st) + (int64_t)rs->ids[r][g] * P) * rb, host_req_off(st, r) + g * page_bytes,
                               page_bytes);
          if (e != HSK_OK) return e;
        }
    }
    hsk_status e = c.flush();
    if (e != HSK_OK) return e;
  }
  // then retire: clear the map entries (after the backups and earlier readers on s) and free the ids
  MapWriter w(st, s);
  for (int32_t i = 0; i < q; ++i) {
    const int32_t r = order[i];
    for (size_t g = 0; g < rs->ids[r].size(); ++g) {
      if (rs->ids[r][g] < 0) continue;
      if (rs->flags[r][g] & kReady) {
        hsk_status e = w.add(r, (int32_t)g, -1);
        if (e != HSK_OK) return e;
      }
      rs->free_ids.push(rs->ids[r][g]);
      rs->ids[r][g] = -1;
      rs->flags[r][g] = kBacked;
      --rs->held;
    }
    if (out) out[i] = r;
  }
  hsk_status e = w.flush();
  if (e != HSK_OK) return e;
  if (n_out) *n_out = q;
  return record_order(st, s);
}

static hsk_status publish_impl(hsk_store* st, hipStream_t s, bool wait, int32_t* n_out) {
  ResidencyState* rs = st->res;
  MapWriter w(st, s);
  int32_t n = 0;
  while (!rs->batches.empty()) {
    ResidencyState::Batch& b = rs->batches.front();
    if (wait) {
      HSK_HIP(hipEventSynchronize(b.ev));
    } else {
      const hipError_t q = hipEventQuery(b.ev);
      if (q == hipErrorNotReady) {
        (void)hipGetLastError();  // not an error: the copies are still in flight
        break;
      }
      if (q != hipSuccess) return HSK_EHIP;
    }
    for (const auto& p : b.pages) {
      if (!rs->admitted[p.r] || rs->seq[p.r] != p.seq || rs->ids[p.r][p.g] != p.id || (rs->flags[p.r][p.g] & kReady))
        continue;  // released or reclaimed while in flight
      rs->flags[p.r][p.g] |= kReady;
      hsk_status e = w.add(p.r, p.g, p.id);
      if (e != HSK_OK) return e;
      ++n;
    }
    rs->spare.push_back(b.ev);
    rs->batches.pop_front();
  }
  hsk_status e = w.flush();
  if (e != HSK_OK) return e;
  if (n_out) *n_out = n;
  return HSK_OK;
}

}  // namespace hsk

using namespace hsk;

extern "C" {

hsk_status hsk_residency_init(hsk_store* st, const hsk_residency_desc* desc, hsk_stream_t stream) {
  if (!st || !desc) return HSK_EINVAL;
  if (st->res) return HSK_ESTATE;
  if (desc->capacity_pages < 0 || desc->reserve_pages < 0 || desc->required_pages < 0 ||
      desc->pages_per_attempt < 0 || desc->optional < 0 || desc->optional > 1)
    return HSK_EINVAL;
  if (desc->optional && (st->d.page_rows == 0 || st->d.opt_pool_pages == 0)) return HSK_EINVAL;
  if ((int64_t)st->d.num_requests * st->max_pages > 0x7fffffffLL) return HSK_EINVAL;
  // the metadata regions of the sources are equally spaced (every source has the same layout)
  int64_t stride = 0;
  if (st->d.num_sources > 1) {
    stride = (char*)st->meta[1].key - (char*)st->meta[0].key;
    for (int32_t k = 1; k < st->d.num_sources; ++k) {
      const SourceMeta &a = st->meta[k - 1], &b = st->meta[k];
      if ((char*)b.key - (char*)a.key != stride || (char*)b.rec - (char*)a.rec != stride ||
          (char*)b.order - (char*)a.order != stride || (char*)b.pt - (char*)a.pt != stride ||
          (char*)b.plan_n - (char*)a.plan_n != stride || (b.opt && (char*)b.opt - (char*)a.opt != stride))
        return HSK_EINVAL;
    }
  }
  ResidencyState* rs = new (std::nothrow) ResidencyState();
  if (!rs) return HSK_ENOMEM;
  st->res = rs;
  rs->cfg = *desc;
  rs->meta_stride = stride;
  const int32_t R = st->d.num_requests;
  rs->admitted.assign(R, 0);
  rs->seq.assign(R, 0);
  rs->ids.assign(R, {});
  rs->flags.assign(R, {});
  for (int64_t i = 0; i < st->d.opt_pool_pages; ++i) rs->free_ids.push((int32_t)i);
  bool ok = hipEventCreateWithFlags(&rs->order_ev, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < kStageSlots; ++i) {
    ok = hipHostMalloc((void**)&rs->stage[i], kStageBytes, hipHostMallocMapped) == hipSuccess &&
         hipEventCreateWithFlags(&rs->stage_ev[i], hipEventDisableTiming) == hipSuccess;
  }
  if (!ok) {
    (void)hipGetLastError();
    residency_destroy(st);
    return HSK_ENOMEM;
  }
  hipStream_t s = (hipStream_t)stream;
  // every slot free: empty metadata, cleared maps, context -1; host bookkeeping to match
  if (wait_write_through(st, s) != HSK_OK) { residency_destroy(st); return HSK_EHIP; }
  for (int32_t k = 0; k < st->d.num_sources; ++k)
    if (launch_init_meta(st->meta[k], R, st->d.hot_slots, st->d.max_ctx, st->max_pages, s) != hipSuccess) {
      residency_destroy(st);
      return HSK_EHIP;
    }
  const int64_t nctx = (int64_t)R * st->d.num_sources;
  hipLaunchKernelGGL(fill_i64_kernel, dim3((unsigned)std::min<int64_t>((nctx + 255) / 256, 1024)), dim3(256), 0, s,
                     st->d_ctx, nctx, (int64_t)-1);
  if (hipGetLastError() != hipSuccess) { residency_destroy(st); return HSK_EHIP; }
  std::fill(st->ctx.begin(), st->ctx.end(), (int64_t)-1);
  std::fill(st->n_import.begin(), st->n_import.end(), (int64_t)0);
  for (auto& v : st->opt_mirror) std::fill(v.begin(), v.end(), -1);
  return HSK_OK;
}

hsk_status hsk_request_admit(hsk_store* st, int32_t req, int64_t n_rows, const void* d_history, int64_t source_stride,
                             hsk_stream_t stream, int32_t* reclaimed, int32_t* n_reclaimed) {
  if (n_reclaimed) *n_reclaimed = 0;
  if (!st || req < 0 || req >= st->d.num_requests || n_rows < 1 || n_rows > st->d.max_ctx || source_stride < 0)
    return HSK_EINVAL;
  ResidencyState* rs = st->res;
  if (!rs || rs->admitted[req]) return HSK_ESTATE;
  const int64_t rb = st->d.row_bytes, P = st->d.page_rows, T = st->d.tail_rows;
  const int64_t stride = source_stride ? source_stride : n_rows * rb;
  if (d_history && st->host_sources > 1 && stride < n_rows * rb) return HSK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  // Eq. 3: the request's required allocation must fit beside the held optional pages and the reserve
  const int64_t need =
      rs->cfg.required_pages * (rs->n_admitted + 1) + rs->held + rs->cfg.reserve_pages - rs->cfg.capacity_pages;
  if (need > 0) {
    hsk_status e = reclaim_impl(st, need, s, reclaimed, n_reclaimed);
    if (e != HSK_OK) return e;
  }
  if (wait_write_through(st, s) != HSK_OK) return HSK_EHIP;
  if (reset_slot(st, req, n_rows, s) != HSK_OK) return HSK_EHIP;
  rs->admitted[req] = 1;
  rs->seq[req] = rs->next_seq++;
  ++rs->n_admitted;
  st->n_import[req] = n_rows;
  const int64_t np = P ? n_rows / P : 0;
  rs->ids[req].assign((size_t)np, -1);
  rs->flags[req].assign((size_t)np, kBacked);
  const int64_t tail_lo = std::max<int64_t>(0, n_rows - T);
  auto tail_runs = [&](Copier& c, int64_t src_base_off) -> hsk_status {
    // positions [tail_lo, n_rows) -> tail ring rows R*B + r*T + (p mod T): at most two contiguous runs
    const int64_t ring0 = (int64_t)st->d.num_requests * st->d.hot_slots + (int64_t)req * T;
    for (int64_t p = tail_lo; p < n_rows;) {
      const int64_t slot = p % T;
      const int64_t cnt = std::min(n_rows - p, T - slot);
      hsk_status e = c.add(src_base_off + p * rb, (ring0 + slot) * rb, cnt * rb);
      if (e != HSK_OK) return e;
      p += cnt;
    }
    return HSK_OK;
  };
  if (d_history) {
    // resident-first: keep complete pages 0, 1, ... on the device while Eq. 3 leaves capacity
    int64_t m = 0;
    if (rs->cfg.optional)
      while (m < np && free_capacity(st) > 0 && !rs->free_ids.empty()) {
        rs->ids[req][m] = rs->free_ids.top();
        rs->free_ids.pop();
        rs->flags[req][m] = kReady;  // ready at once, host backup deferred
        ++rs->held;
        ++m;
      }
    for (int32_t k = 0; k < st->d.num_sources; ++k) {
      const char* src = (const char*)d_history + (int64_t)host_source(st, k) * stride;
      Copier c(rs, s, src, n_rows * rb, pool_of(st, k), pool_bytes(st));
      for (int64_t g = 0; g < m; ++g) {
        hsk_status e = c.add(g * P * rb, (opt_row0(st) + (int64_t)rs->ids[req][g] * P) * rb, P * rb);
        if (e != HSK_OK) return e;
      }
      if (T > 0) {
        hsk_status e = tail_runs(c, 0);
        if (e != HSK_OK) return e;
      }
      hsk_status e = c.flush();
      if (e != HSK_OK) return e;
    }
    // the rest of the history goes to the host rows
    for (int32_t hs = 0; hs < st->host_sources; ++hs) {
      Copier c(rs, s, (const char*)d_history + (int64_t)hs * stride, n_rows * rb, st->host[hs], host_bytes(st));
      hsk_status e = c.add(m * P * rb, host_req_off(st, req) + m * P * rb, (n_rows - m * P) * rb);
      if (e == HSK_OK) e = c.flush();
      if (e != HSK_OK) return e;
    }
    MapWriter w(st, s);
    for (int64_t g = 0; g < m; ++g) {
      hsk_status e = w.add(req, (int32_t)g, rs->ids[req][g]);
      if (e != HSK_OK) return e;
    }
    hsk_status e = w.flush();
    if (e != HSK_OK) return e;
  } else if (T > 0) {
    for (int32_t k = 0; k < st->d.num_sources; ++k) {
      Copier c(rs, s, st->host[host_source(st, k)], host_bytes(st), pool_of(st, k), pool_bytes(st));
      hsk_status e = tail_runs(c, host_req_off(st, req));
      if (e == HSK_OK) e = c.flush();
      if (e != HSK_OK) return e;
    }
  }
  return record_order(st, s);
}

hsk_status hsk_request_release(hsk_store* st, int32_t req, hsk_stream_t stream) {
  if (!st || req < 0 || req >= st->d.num_requests) return HSK_EINVAL;
  ResidencyState* rs = st->res;
  if (!rs || !rs->admitted[req]) return HSK_ESTATE;
  hipStream_t s = (hipStream_t)stream;
  if (wait_pending_of(st, req, s) != HSK_OK || wait_write_through(st, s) != HSK_OK) return HSK_EHIP;
  if (reset_slot(st, req, -1, s) != HSK_OK) return HSK_EHIP;  // clears the slot's optional map too
  for (int32_t id : rs->ids[req])
    if (id >= 0) {
      rs->free_ids.push(id);
      --rs->held;
    }
  rs->ids[req].clear();
  rs->flags[req].clear();
  rs->admitted[req] = 0;
  rs->seq[req] = 0;
  --rs->n_admitted;
  st->n_import[req] = 0;
  return record_order(st, s);
}

hsk_status hsk_residency_reclaim(hsk_store* st, int64_t deficit, hsk_stream_t stream, int32_t* reclaimed,
                                 int32_t* n_reclaimed) {
  if (n_reclaimed) *n_reclaimed = 0;
  if (!st) return HSK_EINVAL;
  if (!st->res) return HSK_ESTATE;
  return reclaim_impl(st, deficit, (hipStream_t)stream, reclaimed, n_reclaimed);
}

hsk_status hsk_residency_publish(hsk_store* st, hsk_stream_t stream, int32_t wait, int32_t* n_published) {
  if (n_published) *n_published = 0;
  if (!st) return HSK_EINVAL;
  if (!st->res) return HSK_ESTATE;
  return publish_impl(st, (hipStream_t)stream, wait != 0, n_published);
}

hsk_status hsk_residency_populate(hsk_store* st, hsk_stream_t stream, hsk_stream_t copy_stream, int32_t* n_reserved) {
  if (n_reserved) *n_reserved = 0;
  if (!st) return HSK_EINVAL;
  ResidencyState* rs = st->res;
  if (!rs) return HSK_ESTATE;
  hsk_status e = publish_impl(st, (hipStream_t)stream, false, nullptr);
  if (e != HSK_OK || !rs->cfg.optional) return e;
  const int32_t R = st->d.num_requests;
  std::vector<ResidencyState::Pending> got;
  int32_t r = rs->cursor, idle = 0;
  while ((int32_t)got.size() < rs->cfg.pages_per_attempt && free_capacity(st) > 0 && !rs->free_ids.empty() &&
         idle < R) {
    int32_t g = -1;
    if (rs->admitted[r])
      for (size_t i = 0; i < rs->ids[r].size(); ++i)
        if (rs->ids[r][i] < 0) { g = (int32_t)i; break; }
    if (g >= 0) {
      const int32_t id = rs->free_ids.top();
      rs->free_ids.pop();
      rs->ids[r][g] = id;  // reserved: pending until its copy completes and it is published
      ++rs->held;
      got.push_back({r, g, id, rs->seq[r]});
      idle = 0;
      rs->cursor = (r + 1) % R;
    } else {
      ++idle;
    }
    r = (r + 1) % R;
  }
  if (got.empty()) return HSK_OK;
  hipStream_t c = (hipStream_t)copy_stream;
  if (rs->order_recorded) HSK_HIP(hipStreamWaitEvent(c, rs->order_ev, 0));
  const int64_t P = st->d.page_rows, rb = st->d.row_bytes;
  for (int32_t k = 0; k < st->d.num_sources; ++k) {
    Copier cp(rs, c, st->host[host_source(st, k)], host_bytes(st), pool_of(st, k), pool_bytes(st));
    for (const auto& p : got) {
      e = cp.add(host_req_off(st, p.r) + (int64_t)p.g * P * rb, (opt_row0(st) + (int64_t)p.id * P) * rb, P * rb);
      if (e != HSK_OK) return e;
    }
    e = cp.flush();
    if (e != HSK_OK) return e;
  }
  hipEvent_t ev = nullptr;
  if (!rs->spare.empty()) {
    ev = rs->spare.back();
    rs->spare.pop_back();
  } else {
    HSK_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  }
  HSK_HIP(hipEventRecord(ev, c));
  rs->batches.push_back({ev, std::move(got)});
  if (n_reserved) *n_reserved = (int32_t)rs->batches.back().pages.size();
  return HSK_OK;
}

hsk_status hsk_residency_query(hsk_store* st, hsk_residency_info* info) {
  if (!st || !info) return HSK_EINVAL;
  const ResidencyState* rs = st->res;
  if (!rs) return HSK_ESTATE;
  hsk_residency_info o{};
  o.admitted = rs->n_admitted;
  o.next_slot = rs->cursor;
  o.required_pages = rs->cfg.required_pages * rs->n_admitted;
  o.optional_pages = rs->held;
  for (int32_t r = 0; r < st->d.num_requests; ++r) {
    if (!rs->admitted[r]) continue;
    o.eligible_pages += (int64_t)rs->ids[r].size();
    for (size_t g = 0; g < rs->ids[r].size(); ++g) {
      if (rs->ids[r][g] >= 0 && (rs->flags[r][g] & kReady)) ++o.ready_pages;
      if (!(rs->flags[r][g] & kBacked)) ++o.unbacked_pages;
    }
  }
  o.pending_pages = o.optional_pages - o.ready_pages;
  o.free_pages = free_capacity(st);
  *info = o;
  return HSK_OK;
}

hsk_status hsk_residency_pages(hsk_store* st, int32_t req, int32_t* ids, uint8_t* flags, int64_t cap,
                               int64_t* n_pages) {
  if (!st || !n_pages || req < 0 || req >= st->d.num_requests || cap < 0) return HSK_EINVAL;
  const ResidencyState* rs = st->res;
  if (!rs) return HSK_ESTATE;
  const int64_t n = (int64_t)rs->ids[req].size();
  *n_pages = n;
  for (int64_t g = 0; g < std::min(n, cap); ++g) {
    if (ids) ids[g] = rs->ids[req][g];
    if (flags) flags[g] = (rs->ids[req][g] >= 0 && (rs->flags[req][g] & kReady) ? kReady : 0) |
                          (rs->flags[req][g] & kBacked);
  }
  return HSK_OK;
}

}  // extern "C"
