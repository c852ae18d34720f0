/*
 * hsk -- hierarchical sparse KV resolve + sparse decode attention for MI355X (gfx950).
 *
 * C ABI of libhsk.so.  Plain pointers and sizes only; every call returns an hsk_status and never throws.
 *
 * What the library does, per decode step and layer (the hot path):
 *   1. hsk_resolve_step: the model's top-k selected positions of each request (logical positions) are
 *      turned into physical rows of a device pool (pool locations), as the fused Resolve kernel of
 *      "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV Cache Management" (section 3.4)
 *      does: tail rows and ready optional-history pages resolve directly ("Adaptive DHiSparse:
 *      Speculative Decoding over a Load-Adaptive KV Hierarchy", section 3.2, Figure 2 callout 1), the
 *      rest are looked up in a per-request hot cache of B slots managed by LRU with hits ranked above the
 *      same step's fills (HiSparse section 3.2), and missing rows are copied from a pinned host-memory
 *      store into LRU victim slots, or into staging rows when a multi-query union overflows the free slots
 *      (Adaptive DHiSparse section 3.3, Eqs. 5-6).  Each distinct missing row is copied once.
 *   2. hsk_sparse_decode_attn: exact softmax attention of each query over the rows at the emitted
 *      locations (MLA: 576-wide rows, keys = row[0:dk], values = row[0:dv]; GQA: 16-token pages).
 *
 * Ownership: the library owns the opaque store and its pinned host KV rows (allocated with hipHostMalloc,
 * freed by hsk_kv_store_destroy).  The caller owns every device buffer (workspace, pool, selections,
 * locations, queries, outputs, statistics, attention scratch) and every stream; device buffers must stay
 * valid until the work queued on them completes.  A store is not thread-safe; calls on one source are
 * ordered by the stream they are issued on.
 *
 * Errors: argument and ordering errors return synchronously and change nothing.  Errors found on the
 * device (a selected position outside [0, n_r): HSK_ERANGE; a multi-query union that overflows staging:
 * HSK_ESTAGE) are written to that request's hsk_stats.status, leave that request's metadata unchanged,
 * set every location of that request to -1, and are also latched in a sticky store word that
 * hsk_sync_status returns and clears.
 */
#ifndef HSK_H
#define HSK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hsk_status;
enum {
  HSK_OK = 0,
  HSK_EINVAL = -1,  /* bad argument or shape */
  HSK_ENOMEM = -2,  /* pinned host allocation failed */
  HSK_EHIP = -3,    /* a HIP runtime call failed */
  HSK_ESTATE = -4,  /* call not valid in the store's state */
  HSK_ERANGE = -5,  /* a selected position is outside [0, n_r) */
  HSK_ESTAGE = -6,  /* a request's missing rows exceed its free hot slots plus its staging rows */
  HSK_EEPOCH = -7,  /* epoch not greater than the last epoch resolved on that source */
  HSK_EWAIT = -8,   /* admission waits: the optional pages cannot cover the capacity it needs */
  HSK_ESCRATCH = -9 /* the call needs more scratch than the library's static buffer holds */
};

/* A hipStream_t, passed as a plain pointer; NULL is the null stream. */
typedef void* hsk_stream_t;

/* Gather modes.  HSK_GATHER_ZEROCOPY: each resolve call ends by copying its misses.  HSK_GATHER_DEFERRED:
 * a resolve call plans only (locations, metadata and the miss plan are final, the missing rows' pool
 * contents are not) and hsk_fetch_plan queues the copy, on a stream of the caller's choice (the plan-then-IO
 * split of HiSparse section 3.5, which lets the copy run beside other work).  HSK_GATHER_NO_IO skips the
 * host reads (the rows left in the slots are stale): it is a timing bound only, like the no-IO oracle of
 * HiSparse section 4.6, and never a correct result. */
enum { HSK_GATHER_ZEROCOPY = 0, HSK_GATHER_NO_IO = 1, HSK_GATHER_DEFERRED = 2 };

/* Limits of this build. */
#define HSK_MAX_HOT_SLOTS 8192
#define HSK_MAX_SELECTIONS_PER_REQUEST 65536

/*
 * Store description.  Sizes are in rows unless noted.  A "row" is what one selected position names: one
 * token's KV record (MLA: 576 bf16 = 1,152 B) or one page of tokens (GQA: 16 tokens x [K|V] = 8,192 B).
 *
 * Per source and request the device pool holds B hot slots, T tail rows and S staging rows; each source
 * also has an optional-history pool of opt_pool_pages pages of page_rows rows.  Pool row layout of one
 * source (row indices are what hsk_resolve_step emits, relative to hsk_pool_base of the source):
 *     hot      r*B + slot                                   r < R, slot < B
 *     tail     R*B + r*T + (p mod T)                        positions p >= n_r - T
 *     optional R*B + R*T + g*page_rows + (p mod page_rows)  page id g of a ready complete page
 *     staging  R*B + R*T + opt_pool_pages*page_rows + r*S + c            (staging_arenas = 0)
 * With staging_arenas = A > 0 the sources share A staging arenas (Adaptive DHiSparse section 3.4: one arena
 * per simultaneously live source, reused by the next layer group once its readers are done): the source
 * regions hold no staging rows, the A arenas of R*S rows follow the last source region, and source s stages
 * into arena s mod A, at relative rows  NS*P_s + (s mod A)*R*S + r*S + c - s*P_s  (P_s = rows of one source
 * region, NS = num_sources).  Sources sharing an arena must be resolved and read in stream order.
 */
typedef struct hsk_desc {
  int32_t num_requests;        /* R: resolution units (requests, or request x KV head for GQA pages) */
  int32_t num_sources;         /* payload sources; each has its own host rows, pool region and metadata */
  int32_t row_bytes;           /* bytes per row; a positive multiple of 16 */
  int32_t hot_slots;           /* B: 1..HSK_MAX_HOT_SLOTS; B >= top_k keeps one query's selection in cache */
  int32_t tail_rows;           /* T >= 0: newest rows of each request, always resident */
  int32_t page_rows;           /* rows per optional-history page; 0 disables optional history */
  int64_t opt_pool_pages;      /* optional-history pages per source (0 if page_rows == 0) */
  int32_t max_queries;         /* Qmax >= 1: queries per request in one resolve call */
  int32_t top_k;               /* k >= 1: selections per query */
  int32_t staging_rows;        /* S >= 0: per request and source */
  int32_t host_alias_sources;  /* 1: every source reads source 0's host rows (one host payload) */
  int64_t max_ctx;             /* rows of host history reserved per request and source */
  const int64_t* ctx_len;      /* host array [R]: n_r at creation (the imported history, every source),
                                  1 <= n_r <= max_ctx, n_r < 2^31; hsk_append_rows grows it per source */
  int32_t gather_mode;         /* HSK_GATHER_ZEROCOPY, HSK_GATHER_NO_IO or HSK_GATHER_DEFERRED */
  int32_t gather_blocks;       /* workgroups (of 16 waves) of the plan copy kernel (hsk_replay_plan,
                                  hsk_fetch_plan); 0 = automatic (32) */
  int32_t staging_arenas;      /* 0: staging inside each source region; A >= 1: A arenas shared by the sources */
} hsk_desc;

/* Per-request result of one resolve call (device memory, written by hsk_resolve_step). */
typedef struct hsk_stats {
  int32_t n_sel;       /* selections examined: nq[r] * k */
  int32_t n_tail;      /* selections resolved from the tail */
  int32_t n_opt;       /* selections resolved from ready optional-history pages */
  int32_t n_hit;       /* distinct hot slots hit */
  int32_t n_hit_sel;   /* selections resolved by hot hits */
  int32_t n_miss;      /* distinct rows copied from host (hot fills + staged) */
  int32_t n_miss_sel;  /* selections resolved by this call's copies */
  int32_t n_staged;    /* distinct rows copied into staging */
  int32_t status;      /* HSK_OK, HSK_ERANGE or HSK_ESTAGE */
  int32_t reserved;
  int64_t fetched_bytes; /* n_miss * row_bytes */
} hsk_stats;

typedef struct hsk_store hsk_store;

/* Device memory the caller must provide for a store described by *desc: the metadata workspace and the
 * row pool of all sources.  Both must be 256-byte aligned.  HiSparse section 3.3 (admission): the
 * per-layer GPU caches of a request (hot slots, tail, staging) are reserved up front, the full history
 * lives in host memory; this call sizes those reservations for all R requests and sources at once. */
hsk_status hsk_workspace_bytes(const hsk_desc* desc, size_t* workspace_bytes, size_t* pool_bytes);

/* HiSparse section 3.3 (admission and prefill): create a store over caller-owned device memory (sizes from
 * hsk_workspace_bytes) and allocate its pinned host rows (num_sources, or 1 with host_alias_sources, x R x max_ctx x row_bytes).  Metadata is set empty
 * on `stream`: keys -1, recency 0, page tables -1, optional maps -1, slot order 0..B-1.  The host rows are
 * uninitialised: the caller writes them (hsk_host_rows) before hsk_commit_prefill.
 * Returns HSK_ENOMEM if the pinned allocation fails. */
hsk_status hsk_kv_store_init(const hsk_desc* desc, void* d_workspace, void* d_pool, hsk_stream_t stream,
                             hsk_store** out);

/* Host pointer to the pinned rows [0, max_ctx) of (source, request); the caller may write them (the
 * prefill stand-in: HiSparse section 3.3 step 1 has prefill write every layer's KV to host memory).  With host_alias_sources every source returns source 0's rows. */
hsk_status hsk_host_rows(hsk_store* store, int32_t source, int32_t req, void** h_rows, int64_t* n_rows);

/* Copy every request's tail rows (positions [n_r - T, n_r)) of every source from host to pool.  HiSparse
 * section 3.3 (1): prefill writes each layer's KV to the host pool; the newest rows stay on device.  Call
 * it once, after the host rows are written and before any append. */
hsk_status hsk_commit_prefill(hsk_store* store, hsk_stream_t stream);

/* Set the optional-history map of complete pages [0, n_pages) of (source, request): h_page_ids[g] is the
 * page id in the source's optional pool (0 <= id < opt_pool_pages), or -1 to drop page g.  Newly mapped
 * pages are copied from host first and their map entries published after the copy, in stream order;
 * dropped entries are cleared in stream order, after earlier readers on the stream (Adaptive DHiSparse
 * section 3.1: ready locations tracked apart from allocated pages, reclaim after earlier readers).
 * Only complete pages of the imported history may be mapped: n_pages <= ctx_len[r] / page_rows (rows
 * generated during decoding stay under the tail and hot-cache rules, section 3.1).  A call that copies
 * rows waits for its copies before returning. */
hsk_status hsk_residency_set(hsk_store* store, int32_t source, int32_t req, const int32_t* h_page_ids,
                             int64_t n_pages, hsk_stream_t stream);

/* Adaptive DHiSparse Eq. 4 (pure host function): walking requests in reclaim order with optional pages
 * h_pages_held[0..n), the smallest q whose first q entries cover `deficit` pages; *q_out = -1 when the
 * optional pages cannot cover it (admission waits), 0 when deficit <= 0. */
hsk_status hsk_reclaim_plan(const int64_t* h_pages_held, int32_t n, int64_t deficit, int32_t* q_out);

/* ---------------------------------------------------------------------------------------------------- */
/* Load-adaptive residency ("Adaptive DHiSparse", section 3.1, Eqs. 3-4)                                */
/* ---------------------------------------------------------------------------------------------------- */
/*
 * After hsk_residency_init the library schedules the optional-history pages itself and requests come and
 * go through hsk_request_admit / hsk_request_release.  Capacity is counted in optional pages (page_rows
 * rows of every source):
 *   Eq. 3   required_pages x (admitted requests) + (optional pages held) + reserve_pages <= capacity_pages,
 * where required_pages stands for one request's required allocation (its hot cache and tail, never lent)
 * and held optional pages are the ready ones plus those whose copies are in flight.  A request's page g
 * (rows [g*page_rows, (g+1)*page_rows) of its imported history, complete pages only) has the same page id
 * in every source's optional pool.  Every row of an admitted request's history is at all times either
 * ready on the device or backed by its host rows, so no resolve ever reads a host row that was not
 * written.
 * Ordering: `stream` is the stream the store's resolves and attention run on.  Map changes (publish and
 * retire) are queued on it, so they take effect after earlier readers on it and before later ones;
 * readers on other streams must be ordered with it by the caller.
 */
typedef struct hsk_residency_desc {
  int64_t capacity_pages;      /* M of Eq. 3 */
  int64_t reserve_pages;       /* M_res of Eq. 3: admission reserve, never lent */
  int64_t required_pages;      /* capacity one admitted request's required allocation takes */
  int32_t pages_per_attempt;   /* bound of one repopulation attempt (hsk_residency_populate) */
  int32_t optional;            /* 1: optional residency on; 0: off (no page is ever held) */
} hsk_residency_desc;

typedef struct hsk_residency_info {
  int32_t admitted;            /* requests admitted */
  int32_t next_slot;           /* where the next round-robin attempt starts */
  int64_t required_pages;      /* required_pages x admitted */
  int64_t optional_pages;      /* pages held: ready + pending */
  int64_t ready_pages;         /* published in the optional maps */
  int64_t pending_pages;       /* reserved, copy in flight or not yet published */
  int64_t unbacked_pages;      /* ready pages whose rows exist only on the device */
  int64_t eligible_pages;      /* complete pages of the admitted requests' imported history */
  int64_t free_pages;          /* capacity optional history may still take under Eq. 3 */
} hsk_residency_info;

/* Page flags reported by hsk_residency_pages. */
enum { HSK_PAGE_READY = 1, HSK_PAGE_BACKED = 2 };

/* Switch the store to scheduled residency: every slot becomes free (context -1: resolves must give it no
 * queries, appends skip it), every optional map is cleared, and hsk_residency_set / hsk_commit_prefill
 * return HSK_ESTATE from then on.  EINVAL for negative sizes, optional = 1 on a store without optional
 * pages; ESTATE if called twice.  Allocates a small pinned staging ring for copy and map lists. */
hsk_status hsk_residency_init(hsk_store* store, const hsk_residency_desc* desc, hsk_stream_t stream);

/*
 * Admission (section 3.1): a new request takes free slot `req` with n_rows (1..max_ctx) of imported
 * history.  If Eq. 3 leaves a deficit, whole requests are reclaimed first (hsk_residency_reclaim, in
 * admission order, oldest first); if all held optional pages cannot cover it the call returns HSK_EWAIT
 * and changes nothing.  The slot's hot cache is reset empty, its context becomes n_rows in every source and
 * its newest tail_rows rows are placed in its tail.
 *   d_history != NULL (resident-first admission): the history is in device memory, source s at
 *     d_history + hs * source_stride bytes, [n_rows][row_bytes], hs = 0 with host_alias_sources else s
 *     (source_stride 0 = n_rows * row_bytes).  While Eq. 3 leaves capacity, complete pages 0, 1, ... are
 *     kept on the device as optional pages (ready at once, host backup deferred); the remaining rows are
 *     written to the host rows.  d_history must stay valid until `stream` passes the call.
 *   d_history == NULL: the caller has already written the host rows (hsk_host_rows); nothing is retained and
 *     pages come later through hsk_residency_populate.  A caller reusing a released slot synchronises
 *     `stream` before writing its host rows.
 * reclaimed (nullable, room for num_requests) receives the reclaimed slots, *n_reclaimed their count.
 * ESTATE if the slot is admitted or residency is not initialised.
 */
hsk_status hsk_request_admit(hsk_store* store, int32_t req, int64_t n_rows, const void* d_history,
                             int64_t source_stride, hsk_stream_t stream, int32_t* reclaimed,
                             int32_t* n_reclaimed);

/* The request in slot `req` finished: its optional pages are retired without backup (its history is no
 * longer needed), queued on `stream` after earlier readers and after any in-flight copy into them; the
 * slot becomes free (context -1).  `stream` is also ordered after the slot's pending write-throughs. */
hsk_status hsk_request_release(hsk_store* store, int32_t req, hsk_stream_t stream);

/* Eq. 4 reclaim: walking the admitted requests in admission order, take every optional page of the first
 * q, q the smallest prefix whose pages cover `deficit`.  Pages whose rows exist only on the device are
 * copied to their host rows first; the map entries are cleared after those copies and after earlier
 * readers (all on `stream`); the page ids are then free for later work on `stream` and for populations.
 * The requests stay admitted (their history is then fetched from host until repopulated).  HSK_EWAIT and
 * no change when all held pages cannot cover the deficit; deficit <= 0 reclaims nothing. */
hsk_status hsk_residency_reclaim(hsk_store* store, int64_t deficit, hsk_stream_t stream, int32_t* reclaimed,
                                 int32_t* n_reclaimed);

/* One bounded round-robin repopulation attempt (section 3.1).  First publishes the pending pages whose
 * copies have completed (hsk_residency_publish with wait = 0).  Then, while Eq. 3 leaves capacity and page
 * ids are free, visits admitted slots round-robin from where the last attempt stopped, reserving for each
 * visited request its lowest-numbered page not held (one page per visit, lowest free page id), up to
 * pages_per_attempt pages.  Their rows are copied from the host rows into the optional pools on
 * `copy_stream` (which first waits for earlier admissions, releases and reclaims on `stream`); the pages
 * stay pending (unmapped) until published.  *n_reserved = pages reserved. */
hsk_status hsk_residency_populate(hsk_store* store, hsk_stream_t stream, hsk_stream_t copy_stream,
                                  int32_t* n_reserved);

/* Publish ready locations: the pending pages whose copies have completed (wait = 1: wait for all of them)
 * enter the optional maps, queued on `stream`.  *n_published (nullable) = pages published. */
hsk_status hsk_residency_publish(hsk_store* store, hsk_stream_t stream, int32_t wait, int32_t* n_published);

/* Host-side view of the scheduler (no device work). */
hsk_status hsk_residency_query(hsk_store* store, hsk_residency_info* info);

/* Per-page state of the request in slot `req`: ids[g] (page id or -1) and flags[g] (HSK_PAGE_READY |
 * HSK_PAGE_BACKED) for its complete pages g < *n_pages (at most cap written; either pointer may be NULL). */
hsk_status hsk_residency_pages(hsk_store* store, int32_t req, int32_t* ids, uint8_t* flags, int64_t cap,
                               int64_t* n_pages);

/*
 * One resolve call on `source` at LRU clock `epoch` (strictly increasing per source; EEPOCH otherwise).
 *   d_sel   int32 [R][Qmax][k] device: query j of request r uses d_sel[r][j][0..k) when j < nq[r]
 *   d_nq    int32 [R] device queries per request (1..Qmax), or NULL for Qmax everywhere
 *   d_locs  int32 [R][Qmax][k] device out: pool row of every selection, in selection order (-1 for
 *           queries j >= nq[r] and for rejected requests)
 *   d_stats hsk_stats [R] device out, or NULL
 * Queued on `stream`: one resolve kernel, one workgroup per request, which ends by copying its request's
 * distinct missing rows from pinned host memory into their slots with 16-byte zero-copy loads (none with
 * HSK_GATHER_NO_IO or HSK_GATHER_DEFERRED).  Locations and pool rows are final when the stream reaches the
 * end of the call (with HSK_GATHER_DEFERRED, the pool rows of the misses once hsk_fetch_plan's copy is
 * done).  The distinct missing rows and their destination rows are kept as the source's miss plan
 * (HiSparse section 3.5) until its next resolve call.
 */
hsk_status hsk_resolve_step(hsk_store* store, int32_t source, uint32_t epoch, const int32_t* d_sel,
                            const int32_t* d_nq, int32_t* d_locs, hsk_stats* d_stats, hsk_stream_t stream);

/*
 * Decode-loop append (HiSparse section 3.3, step 4: newly generated KV written through to host; Adaptive DHiSparse
 * section 3.2, the tail): every request of `source` takes `count` new rows, d_rows [R][count][row_bytes]
 * (device, e.g. the layer's KV of the tokens just generated), as positions n_r .. n_r + count - 1.
 *   On `stream`: the rows are written into the request's tail ring (pool row R*B + r*T + (p mod T)) and
 *   n_r grows, so the newest positions resolve directly for the following resolve calls; the row that
 *   leaves the tail (position n_r - T) becomes history, resolved through the hot cache and fetched from
 *   its host copy.
 *   On `backup_stream` (may equal `stream`): after an event on `stream`, the new rows are written through
 *   from the tail ring to the pinned host rows [r][n_r ..].  The stream waits for that copy at the
 *   second-next append of the source, which is also the first after which those rows can leave the tail
 *   (2 count <= T), so the host copy is complete before any fetch can reference it.
 * d_rows may be reused once `stream` passes the call.  EINVAL (nothing queued): count < 1, 2 count > T,
 * n_r + count > max_ctx for some request, or a store with host_alias_sources.
 */
hsk_status hsk_append_rows(hsk_store* store, int32_t source, const void* d_rows, int32_t count,
                           hsk_stream_t stream, hsk_stream_t backup_stream);

/* Rows of (source, request) context after the appends issued so far (host bookkeeping, no device access). */
hsk_status hsk_context_rows(hsk_store* store, int32_t source, int32_t req, int64_t* n_rows);

/* Adaptive DHiSparse Eq. 8 (pure host function): for a source that packs m consecutive token positions into
 * each stored row, the rows completed when a request's tokens grow from n_before to n_after are
 * [first, first + count) with first = floor(n_before / m) and first + count = floor(n_after / m); a
 * partly filled last row is not counted and remains a tail row. */
hsk_status hsk_completed_rows(int64_t n_before, int64_t n_after, int32_t m, int64_t* first, int64_t* count);

/*
 * Draft KV ring (Adaptive DHiSparse section 3.4, Eqs. 9-10).  A drafter that reads at most `window` prior
 * positions plus its current block of at most k_max positions keeps, per request slot i, a ring of
 *     R_d = page_rows * ceil((window + page_rows - 1 + k_max) / page_rows)      rows (Eq. 9),
 * and draft position t of slot i lives at ring row  phi(i, t) = i * R_d + (t mod R_d)  (Eq. 10): within a
 * slot, positions that are live together map to distinct rows, and each slot owns its own R_d rows.  The ring is caller-owned device
 * memory of slots * R_d rows; hsk_sparse_decode_attn over hsk_ring_window_locs is the drafter's attention.
 */
hsk_status hsk_ring_rows(int64_t window, int32_t page_rows, int32_t k_max, int64_t* ring_rows);

/* Write `count` new draft rows of every slot: d_rows [slots][count][row_bytes] (device) go to ring rows
 * phi(i, d_t0[i] + j), j < count, of d_ring; d_t0 int64 [slots] (device) is each slot's first new position.
 * EINVAL for count < 1, a ring smaller than count rows, or row_bytes not a positive multiple of 16. */
hsk_status hsk_ring_write(void* d_ring, int64_t ring_rows, int32_t slots, const void* d_rows, int32_t count,
                          int32_t row_bytes, const int64_t* d_t0, hsk_stream_t stream);

/* Locations of the window the drafter reads: d_locs int32 [slots][window] gets phi(i, d_t_end[i] - window + j),
 * positions d_t_end[i] - window .. d_t_end[i] - 1 in order, and -1 for positions below 0 (a window not yet
 * full; such entries must not be passed to attention).  EINVAL if window > ring_rows or slots * ring_rows
 * exceeds the int32 row range. */
hsk_status hsk_ring_window_locs(int64_t ring_rows, int32_t slots, int32_t window, const int64_t* d_t_end,
                                int32_t* d_locs, hsk_stream_t stream);

/* Plan replay (HiSparse section 3.5, plan-then-IO): copy the rows listed in plan_source's last miss plan
 * from dst_source's host rows into dst_source's pool, at the same pool rows (EINVAL for a store with shared
 * staging arenas and staging rows, whose staged rows are not at the same relative rows, and for
 * plan_source == dst_source).  A layer that shares its anchor's selection then reads its own payload at the
 * anchor's locations.  Order it after the anchor's resolve and before the consumer's attention with events
 * when it runs on a side stream.
 * A replay destination is replay-only: its pool rows follow plan_source's slot table while its own metadata
 * stays empty, so once a source has received a replay, hsk_resolve_step and hsk_resolve_attend on it return
 * HSK_ESTATE, and so does a replay into a source that has resolved before or from a source that is itself a
 * replay destination. */
hsk_status hsk_replay_plan(hsk_store* store, int32_t plan_source, int32_t dst_source, hsk_stream_t stream);

/* Deferred fetch (HiSparse section 3.5, plan-then-IO; section 3.4 phase 4, the copy by GPU threads): queue on
 * `stream` the copy of `source`'s last miss plan, the distinct rows its last hsk_resolve_step found missing,
 * from the source's pinned host rows into the pool rows that call emitted for them.  For stores in
 * HSK_GATHER_DEFERRED mode, whose resolve calls do not copy.  The copy kernel runs gather_blocks workgroups
 * of 16 waves (0 = automatic: 32), spread evenly over the plan's rows; 16 of them fill the host link and
 * leave the other compute units to work on other streams meanwhile.
 * Ordering is the caller's: queue it after the resolve (same stream, or an event), make readers of the
 * rows (attention) wait for it, and order the source's next resolve call after it (that call rewrites the
 * plan and may evict the slots being filled).  EINVAL: bad source or a store in another gather mode;
 * ESTATE: no resolve on that source yet, or a replay destination. */
hsk_status hsk_fetch_plan(hsk_store* store, int32_t source, hsk_stream_t stream);


/*
 * Promotion copy-back ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", section
 * 3.4 and Figure 3 callout 3: staged rows that are promoted are copied back to stable hot-cache addresses
 * before the staging arena is reused).  The pages leave open which rows are promoted; this call ties it to
 * the round's acceptance (Eq. 7): queries 0..d_accepted[r] of request r are committed (the anchor and its
 * accepted drafts; values are clamped to [0, nq[r] - 1]), the others rejected.  After the source's last
 * hsk_resolve_step (epoch e):
 *   - the staged rows that a committed query selected, in staging order, and not already in the hot cache,
 *   - take the hot slots touched at epoch e whose rows no committed query selected, in ascending
 *     (recency, slot) order (rows only rejected drafts asked for; this epoch's fills before its hits),
 * pairwise, as many as both lists allow: the slot's old position leaves the cache, the staged row becomes a
 * fill of epoch e, and its bytes are copied on the device from its staging row into the slot's pool row (no
 * host read).  The next resolve then finds committed rows hot instead of fetching them from host again.
 *   d_locs:     the int32 [R][Qmax][k] locations that the last hsk_resolve_step on `source` emitted.
 *   d_nq:       int32 [R] query counts of that call, or NULL (all Qmax).
 *   d_accepted: int32 [R] accepted drafts per request.
 *   d_promoted: int32 [R] rows promoted per request (device), or NULL.
 * Order it after the round's attention on `source` (it overwrites hot rows that rejected drafts read) and
 * before the next resolve on `source` or on a source sharing its staging arena.  A second call after the same
 * resolve promotes nothing.  HSK_ESTATE if the source has not resolved yet or is a replay destination;
 * HSK_EINVAL if staging_rows exceeds HSK_MAX_SELECTIONS_PER_REQUEST.
 */
hsk_status hsk_promote_staged(hsk_store* store, int32_t source, const int32_t* d_locs, const int32_t* d_nq,
                              const int32_t* d_accepted, int32_t* d_promoted, hsk_stream_t stream);

/* Device address of a source's pool region (row 0 of the layout above). */
hsk_status hsk_pool_base(hsk_store* store, int32_t source, void** d_pool_source);

/* ---------------------------------------------------------------------------------------------------- */
/* Sparse decode attention                                                                              */
/* ---------------------------------------------------------------------------------------------------- */
enum { HSK_ATTN_MLA = 0, HSK_ATTN_GQA = 1 };

typedef struct hsk_attn_desc {
  int32_t kind;          /* HSK_ATTN_MLA or HSK_ATTN_GQA */
  int32_t num_requests;  /* MLA: R.  GQA: requests (units = requests x kv_heads) */
  int32_t max_queries;   /* MLA: Qmax.  GQA: 1 */
  int32_t heads;         /* MLA: query heads sharing the latent row.  GQA: query heads per request */
  int32_t kv_heads;      /* MLA: 1.  GQA: KV heads; q head h reads KV head h / (heads / kv_heads) */
  int32_t dk;            /* MLA: key width (row[0:dk]).  GQA: head dim */
  int32_t dv;            /* MLA: value width (row[0:dv], dv <= dk).  GQA: head dim (= dk) */
  int32_t top_k;         /* selected rows (MLA) or pages (GQA) per query */
  int32_t row_elems;     /* bf16 values per pool row (MLA >= dk; GQA page_tokens * 2 * dk) */
  int32_t page_tokens;   /* GQA: tokens per page row, each [K dk | V dk].  MLA: 1 */
  int32_t split;         /* partitions of the k rows per query (split-k); 0 = automatic.  A forced split is
                            an upper bound: partitions hold ceil(k / split) rows each and only the non-empty
                            ones, ceil(k / ceil(k / split)) of them, are made */
  float scale;           /* softmax scale, e.g. 1/sqrt(dk); must be positive and finite (else HSK_EINVAL) */
} hsk_attn_desc;

/* Device scratch (bytes) that hsk_sparse_decode_attn and hsk_resolve_attend need for split-k partial
 * results. */
hsk_status hsk_attn_scratch_bytes(const hsk_attn_desc* desc, size_t* scratch_bytes);

/*
 * out = softmax(scale * q . K^T) V over the rows at d_locs, bf16 in, fp32 accumulation, bf16 out
 * (Adaptive DHiSparse Eq. 1; section 3.5: the rows are the model's selected rows, so the result equals
 * attention over a fully resident cache at the same indices).
 *   MLA: d_q bf16 [R][Qmax][H][dk]; d_locs int32 [R][Qmax][k]; d_out bf16 [R][Qmax][H][dv];
 *        d_nq int32 [R] or NULL (queries j >= nq[r] are skipped and their outputs left untouched).
 *   GQA: d_q bf16 [R][H][dk]; d_locs int32 [R * kv_heads][k] (page rows); d_out bf16 [R][H][dk].
 *   d_pool: row 0 of the source's pool (hsk_pool_base); every non-negative location must be a valid row of
 *           it.  A negative location (the -1 that hsk_resolve_step writes for every selection of a request it
 *           rejects) is read as row 0: the query's output is then meaningless, but no load leaves the pool.
 *   d_scratch: at least hsk_attn_scratch_bytes bytes, 256-byte aligned.
 */
hsk_status hsk_sparse_decode_attn(const hsk_attn_desc* desc, const void* d_q, const void* d_pool,
                                  const int32_t* d_locs, const int32_t* d_nq, void* d_out, void* d_scratch,
                                  size_t scratch_bytes, hsk_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): hsk_sparse_decode_attn with its split-k scratch taken from a static
 * device buffer inside the library instead of a caller buffer.  Same kernels, partitions and results as
 * hsk_sparse_decode_attn with the same descriptor.  The buffer holds HSK_NOALLOC_SCRATCH_BYTES bytes on
 * every GPU the library runs on and lives until the process ends; its device address is looked up once
 * per device on the first call there (with that device current).  The call allocates nothing.
 *   The device is the one current at the call; `stream` must belong to it.
 *   Every call on one GPU shares that GPU's buffer, which keeps the last call's contents: calls that can
 *   overlap on one GPU (different streams without ordering between them) race and give wrong results;
 *   order them on one stream or with events.
 * HSK_ESCRATCH (nothing queued) if hsk_attn_scratch_bytes(desc) exceeds HSK_NOALLOC_SCRATCH_BYTES; other
 * errors as hsk_sparse_decode_attn.
 */
#define HSK_NOALLOC_SCRATCH_BYTES (64u << 20)
hsk_status hsk_sparse_decode_attn_noalloc(const hsk_attn_desc* desc, const void* d_q, const void* d_pool,
                                          const int32_t* d_locs, const int32_t* d_nq, void* d_out,
                                          hsk_stream_t stream);

/*
 * Resolve (HiSparse section 3.4) and MLA sparse decode attention (Adaptive DHiSparse Eq. 1) in one call,
 * for stores with max_queries = 1 in HSK_GATHER_ZEROCOPY mode.  The attention kernel reads the rows this
 * call fetches straight from the pinned host rows and writes each of them once into its pool row, so the
 * host reads overlap the attention over resident rows instead of preceding it (the overlap of IO with
 * computation of HiSparse section 3.5, within one layer).  Locations, statistics, pool contents and the
 * miss plan are those of hsk_resolve_step; d_out is attention over the same rows as hsk_sparse_decode_attn
 * with the same partitions (whenever hsk_sparse_decode_attn's partitions hold at most 1,024 rows), equal to
 * it bit for bit when the heads are not a multiple of 64 (both then run the same kernel) and within bf16
 * rounding otherwise (hsk_sparse_decode_attn then runs its 32-heads-per-wave kernel, which sums in another
 * order).
 *   d_sel, d_locs, d_stats: as hsk_resolve_step with Qmax = 1 (no query counts).
 *   desc: an HSK_ATTN_MLA descriptor with num_requests, top_k and row_elems * 2 equal to the store's
 *         requests, top_k and row_bytes, row_elems = dk, max_queries = 1; its partitions hold at most
 *         1,024 rows.
 *   d_q, d_out, d_scratch, scratch_bytes: as hsk_sparse_decode_attn (hsk_attn_scratch_bytes covers both).
 * EINVAL (nothing queued) for another store or descriptor shape, or max_ctx >= 2^30; EEPOCH as
 * hsk_resolve_step.  Outputs of a request that the resolve rejects (status in its stats) are NaN.
 */
hsk_status hsk_resolve_attend(hsk_store* store, int32_t source, uint32_t epoch, const int32_t* d_sel,
                              int32_t* d_locs, hsk_stats* d_stats, const hsk_attn_desc* desc, const void* d_q,
                              void* d_out, void* d_scratch, size_t scratch_bytes, hsk_stream_t stream);

/*
 * A stream with a hardware queue of its own, for the streams of an overlapped schedule (the copy stream and each
 * micro-batch's stream of hsk_resolve_fetch_attend).  The HIP runtime serves ordinary streams from a small pool of
 * hardware queues, handed out in turn as streams are created; two streams on one queue run as one FIFO, so a
 * fetch queued behind another stream's attention waits for it and the overlap is lost.  A stream created with a
 * compute-unit mask gets a queue of its own; this one enables every compute unit of the current device, so it
 * runs like any other stream (default priority).  The caller destroys it with hsk_stream_destroy.
 * EHIP if the runtime refuses. */
hsk_status hsk_stream_create(hsk_stream_t* stream);
hsk_status hsk_stream_destroy(hsk_stream_t stream);

/*
 * One layer of a deferred store with its host IO overlapped (HiSparse section 3.5: plan, then IO beside other
 * work; Adaptive DHiSparse Eq. 1 attention over the resolved rows).  Queues, in order:
 *   on `stream`       the resolve of hsk_resolve_step (plan only); each of its workgroups then publishes its
 *                     request's plan by storing `epoch` in the store's per-request ready word;
 *   on `copy_stream`  the fetch of hsk_fetch_plan, whose kernel waits inside, per request, for that word to
 *                     read `epoch` before it reads the plan; its launch records the store's event for the
 *                     source when the kernel ends;
 *   on `stream`       a wait for the fetch, then hsk_sparse_decode_attn(desc, d_q, pool of `source`, d_locs, d_nq,
 *                     d_out, d_scratch, scratch_bytes).
 * While the copy stream streams this source's missing rows over the host link, the caller's other streams (other
 * micro-batches, other work) run; the attention starts when its rows are in.  Calls for different stores or
 * sources sharing one copy stream are fetched in call order, one at a time, with no cross-stream wait between
 * consecutive fetches (such a wait costs several microseconds of idle link each).  A fetch that sees no plan
 * for a request within seconds copies nothing for it and records HSK_ESTATE in the store's error word
 * (hsk_sync_status); it cannot happen through these calls alone, since every call queues its resolve before its
 * fetch and fetches run in call order.  copy_stream may equal stream (plain stream order then, no waits).  The
 * event belongs to the store, one per source.  The source's next call comes after this one's fetch when it is
 * queued on the same `stream` (its attention waits for the fetch); on another stream the caller orders it after
 * this call's attention.
 *   d_sel, d_nq, d_locs, d_stats, epoch: as hsk_resolve_step.
 *   desc: any attention descriptor whose resolution units (num_requests; num_requests x kv_heads for
 *         HSK_ATTN_GQA), max_queries and top_k equal the store's requests, max_queries and top_k, and with
 *         row_elems * 2 = row_bytes; d_q, d_out, d_scratch, scratch_bytes as hsk_sparse_decode_attn.
 * EINVAL (nothing queued): a store not in HSK_GATHER_DEFERRED mode, a descriptor hsk_sparse_decode_attn would
 * reject or that does not match the store, too small or misaligned scratch; ESTATE for a replay destination;
 * EEPOCH as hsk_resolve_step.  Outputs of a request the resolve rejects (status in its stats) are meaningless:
 * its locations are -1, which the attention reads as row 0.
 */
hsk_status hsk_resolve_fetch_attend(hsk_store* store, int32_t source, uint32_t epoch, const int32_t* d_sel,
                                    const int32_t* d_nq, int32_t* d_locs, hsk_stats* d_stats,
                                    const hsk_attn_desc* desc, const void* d_q, void* d_out, void* d_scratch,
                                    size_t scratch_bytes, hsk_stream_t stream, hsk_stream_t copy_stream);

/* ---------------------------------------------------------------------------------------------------- */
/* Inspection (tests) and lifetime                                                                     */
/* ---------------------------------------------------------------------------------------------------- */
/* Synchronous copy of (source, request) metadata into caller host buffers (any may be NULL):
 * key[B] (position held, -1 empty), rec[B] (2e+1 after a hit at epoch e, 2e after a fill, 0 empty),
 * order[B] (slots in ascending (rec, slot) order), pt[n_r] (slot of a position or -1; n_r of the source
 * after its appends, hsk_context_rows), opt[ctx_len[r] / page_rows] (optional page id or -1).  Waits for all
 * work on the device. */
hsk_status hsk_snapshot(hsk_store* store, int32_t source, int32_t req, int32_t* key, uint32_t* rec,
                        uint16_t* order, int32_t* pt, int32_t* opt);

/* Synchronous copy of (source, request)'s last miss plan: *n distinct missing positions in miss order
 * (first occurrence over the flattened query lists) and the pool row each was copied to; at most cap
 * entries are written. */
hsk_status hsk_read_plan(hsk_store* store, int32_t source, int32_t req, int32_t* pos, int32_t* dst, int32_t cap,
                         int32_t* n);

/* Wait for `stream`, then return and clear the first device-side error latched since the last call. */
hsk_status hsk_sync_status(hsk_store* store, hsk_stream_t stream);

/* Free the pinned host rows and the store (device memory stays with the caller).  Waits for the device. */
void hsk_kv_store_destroy(hsk_store* store);

const char* hsk_status_str(hsk_status status);

#ifdef __cplusplus
}
#endif

#endif /* HSK_H */
