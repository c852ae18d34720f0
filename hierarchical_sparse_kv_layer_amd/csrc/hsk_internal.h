// Internal declarations shared by the host runtime and the kernels of libhsk.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "hsk.h"

#define HSK_HIP(call)                                   \
  do {                                                  \
    hipError_t hsk_e_ = (call);                         \
    if (hsk_e_ != hipSuccess) return HSK_EHIP;          \
  } while (0)

namespace hsk {

constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / 64;
constexpr int kGatherThreads = 256;
// The plan copy kernel: a compute unit's host-read rate grows with the waves it runs (one wave ~0.7 GB/s,
// four ~1.5, sixteen ~3.4 GB/s) whatever each wave keeps in flight, so its workgroups are 16 waves and 16-18 of
// them fill the host link while leaving the other compute units free.
constexpr int kFetchThreads = 1024;
constexpr int64_t kAlign = 256;
// A copy kernel that waits inside for a plan published by a resolve on another stream gives up after this many
// polls of a request's ready word (each a device-scope load and a short sleep: seconds in all).
constexpr uint32_t kPlanSpinLimit = 1u << 22;

// Device pointers of one source's metadata (all inside the caller's workspace).
struct SourceMeta {
  int32_t* key;       // [R][B] position held by a hot slot, -1 empty
  uint32_t* rec;      // [R][B] recency stamp: 2e+1 hit, 2e fill, 0 empty
  uint16_t* order;    // [R][B] slots in ascending (rec, slot) order
  int32_t* pt;        // [R][max_ctx] page table: slot of a position, or -1 (transiently: claims/staging codes)
  int32_t* opt;       // [R][max_pages] optional page id of a complete page, or -1 (null without pages)
  int32_t* plan_n;    // [R] distinct missing rows of the last resolve call
  int32_t* plan_pos;  // [R][plan_cap] their positions, in miss order
  int32_t* plan_dst;  // [R][plan_cap] the pool row each was copied to
  uint32_t* ready;    // [R] epoch of the last resolve that published its plan here (0: none)
};

// Byte offsets of every region of the workspace.
struct WorkspaceLayout {
  int64_t ctx, wt_pos, err, fill, total;   // ctx [S][R] i64, wt_pos [S][2][R] i32
  std::vector<int64_t> key, rec, order, pt, opt, plan_n, plan_pos, plan_dst, ready;
};

bool layout_workspace(const hsk_desc& d, WorkspaceLayout* out);
int64_t rows_per_source(const hsk_desc& d);
int64_t total_pool_rows(const hsk_desc& d);
int64_t stg_base_of(const hsk_desc& d, int32_t source);

struct ResolveArgs {
  const int32_t* sel;
  const int32_t* nq;
  int32_t* locs;
  hsk_stats* stats;
  const int64_t* ctx;
  SourceMeta m;
  int32_t* err;
  int64_t max_ctx;
  int64_t max_pages;
  int64_t opt_base;   // first optional row: R*B + R*T
  int64_t stg_base;   // first staging row: R*B + R*T + opt_pool_pages*page_rows
  int32_t* fill;       // nullable: per-selection host source for a fused resolve + attend (see resolve.hip)
  const char* host;    // nullable: host rows of (host source, request 0); set, the kernel copies the misses
  char* pool;          // row 0 of the source's pool (the copies' destination)
  int64_t host_req_stride;  // bytes between requests in the host rows
  uint32_t* ready;     // nullable: each workgroup stores epoch in ready[r] once its request's plan is visible
  int32_t plan_cap;
  int32_t R, B, T, P, S, Qmax, k, row_bytes;
  uint32_t epoch;
};

struct GatherArgs {
  const char* host;        // device-visible address of host rows of (host source, request 0)
  char* pool;              // row 0 of the destination source's pool
  const int32_t* plan_n;
  const int32_t* plan_pos;
  const int32_t* plan_dst;
  int64_t host_req_stride; // bytes between requests in the host rows
  const uint32_t* ready;   // nullable: wait in the kernel until ready[r] == epoch before reading request r's plan
  int32_t* err;            // with ready: the store's error word (HSK_ESTATE when a plan never appears)
  uint32_t epoch;
  int32_t plan_cap;
  int32_t row_bytes;
};

struct CopyRun {           // one contiguous byte run, host -> pool
  int64_t src;             // byte offset from the host source base
  int64_t dst;             // byte offset from the pool source base
  int64_t bytes;
};

hipError_t launch_init_meta(const SourceMeta& m, int32_t R, int32_t B, int64_t max_ctx, int64_t max_pages,
                            hipStream_t s);
hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& g, int32_t R, int32_t blocks, hipStream_t s, hipEvent_t done = nullptr);
hipError_t launch_promote(const int32_t* locs, const int32_t* nq, const int32_t* accepted, int32_t* promoted,
                          const SourceMeta& m, char* pool, int64_t max_ctx, int64_t stg_base, int32_t R, int32_t B,
                          int32_t S, int32_t Qmax, int32_t k, int32_t row_bytes, uint32_t epoch, hipStream_t s);
hipError_t launch_tail_copy(const char* host, int64_t host_req_stride, char* pool, const int64_t* d_ctx,
                            int32_t R, int32_t B, int32_t T, int32_t row_bytes, hipStream_t s);
hipError_t launch_copy_runs(const char* host, char* pool, const CopyRun* runs, int32_t n, hipStream_t s);
// decode-loop append: rows -> tail ring, context grows (stream); tail ring -> host rows (backup stream)
hipError_t launch_append_tail(const char* rows, char* pool, int64_t* ctx, int32_t* wt_pos, int32_t R, int32_t B,
                              int32_t T, int32_t count, int32_t row_bytes, hipStream_t s);
hipError_t launch_ring_write(char* ring, int64_t ring_rows, int32_t slots, const char* rows, int32_t count,
                             int32_t row_bytes, const int64_t* t0, hipStream_t s);
hipError_t launch_ring_locs(int64_t ring_rows, int32_t slots, int32_t window, const int64_t* t_end, int32_t* locs,
                            hipStream_t s);
hipError_t launch_write_through(const char* pool, char* host, int64_t host_req_stride, const int32_t* wt_pos,
                                int32_t R, int32_t B, int32_t T, int32_t count, int32_t row_bytes, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// MLA attention that reads the rows this call fetches straight from pinned host memory (fill codes of the
// resolve kernel) and writes each of them once into its pool row; defined in attention.hip.
hsk_status check_mla_fused(const hsk_attn_desc* d, const void* scratch, size_t scratch_bytes);
hsk_status launch_mla_fused(const hsk_attn_desc* d, const void* q, const char* pool, const int32_t* locs,
                            const int32_t* fill, const char* host, int64_t host_req_stride, void* out,
                            void* scratch, size_t scratch_bytes, hipStream_t s);

struct ResidencyState;                       // scheduled residency (residency.hip)
void residency_destroy(hsk_store* st);

}  // namespace hsk

struct hsk_store {
  hsk_desc d;
  std::vector<int64_t> ctx;                 // [source * R + r] rows of each request's context, per source
  std::vector<int64_t> n_import;            // [R] imported (prefill) history: what optional pages may cover
  int64_t max_pages = 0;
  int32_t plan_cap = 0;
  int64_t rows_per_src = 0;
  int32_t host_sources = 0;
  int32_t device = 0;
  char* ws = nullptr;
  char* pool = nullptr;
  int64_t* d_ctx = nullptr;                 // [S][R]
  int32_t* d_wt_pos = nullptr;              // [S][2][R] first position of the last two appends per source
  std::vector<hipEvent_t> wt_done;          // [S][2] write-through of the last two appends per source
  std::vector<uint8_t> wt_pending;          // [S][2] event recorded and not yet waited for
  std::vector<hipEvent_t> tail_done;        // [S] tail writes of the last append
  std::vector<hipEvent_t> fetched;          // [S] the fetch of hsk_resolve_fetch_attend done on the copy stream
  std::vector<int32_t> append_parity;       // [S]
  int32_t* d_err = nullptr;
  int32_t* d_fill = nullptr;                // [R][Qmax][k] per-selection host source of a fused call
  std::vector<hsk::SourceMeta> meta;
  std::vector<char*> host;                  // pinned host rows per host source
  std::vector<uint32_t> last_epoch;         // per source
  std::vector<uint8_t> replay_dst;           // per source: 1 once it received a replayed plan (no own resolves)
  std::vector<std::vector<int32_t>> opt_mirror;  // [source * R + r] host copy of the optional map
  void* h_stage = nullptr;                  // pinned staging for map and run-list uploads
  size_t h_stage_bytes = 0;
  void* d_stage = nullptr;                  // device copy of run lists
  size_t d_stage_bytes = 0;
  hsk::ResidencyState* res = nullptr;       // set by hsk_residency_init: the library schedules residency
};
