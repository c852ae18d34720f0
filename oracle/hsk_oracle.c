/*
 * CPU oracle of the hierarchical sparse KV hot path -- TEST INFRASTRUCTURE ONLY (see hsk_oracle.h).
 *
 * Written for readability, not speed: scalar loops, one request at a time, a full sort for victim choice.
 * Every function names the passage of the pages it follows:
 *   [HS]  "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV Cache Management"
 *   [AD]  "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy"
 *
 * Readings where the pages leave a step open (each is also listed with the design notes):
 *   - recency: rec = 2e+1 for a hit at epoch e, 2e for a fill at epoch e, 0 for an empty slot, so hits
 *     rank just above the same step's fills ([HS] 3.2 "Replacement policy", 3.4 phase 3);
 *   - victims: the non-hit slots in ascending (rec, slot) order; the i-th distinct miss (first
 *     occurrence order over the flattened query lists) takes the i-th victim;
 *   - precedence tail > optional history > hot cache ([AD] 3.2, Figure 2 callout order; a row may be in
 *     the optional map and the hot cache at once, [AD] 3.1);
 *   - directly resolved rows leave the hot-cache metadata untouched ([AD] 3.2: they never reach
 *     replacement);
 *   - misses beyond the free hot slots of a call go to staging in miss order ([AD] 3.3 overflow to
 *     staging); the resolve itself never promotes them: ora_promote, called after the round's acceptance,
 *     copies staged rows of committed queries into slots that only rejected drafts used ([AD] 3.4, Figure 3
 *     callout 3; the reading is stated at ora_promote);
 *   - out-of-range positions and staging overflow reject the whole request before any state changes.
 */
#include "hsk_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

struct ora_source {
  int32_t R, B, T, P, S, row_bytes;
  int64_t opt_pool_pages;
  int64_t* ctx;       /* [R] rows of the context, grown by appends */
  int64_t* n_import;  /* [R] imported history (context at creation or admission) */
  int64_t* uid;       /* [R] identity of the request in each slot (the slot index until an admission) */
  int64_t max_ctx;    /* rows reserved per request */
  int32_t* key;       /* [R][B] position held by a hot slot, -1 = empty */
  uint32_t* rec;      /* [R][B] recency stamp, 0 = empty */
  int32_t** pt;       /* [R] -> [ctx_r] page table: hot slot of a position or -1 */
  int32_t** opt;      /* [R] -> [ctx_r / P] optional page id of a complete page or -1 */
  uint32_t last_epoch;
  int64_t stg_base;   /* first staging row, relative to the source's pool rows */
  int64_t pool_rows;
  int64_t* pool;      /* [pool_rows] pool model: r * 2^32 + position, or -1 */
};

/* pool row addresses, one pool per source (region order: hot, tail, optional, staging) */
static int64_t hot_loc(const ora_source* s, int32_t r, int32_t slot) { return (int64_t)r * s->B + slot; }
static int64_t tail_loc(const ora_source* s, int32_t r, int64_t p) {
  return (int64_t)s->R * s->B + (int64_t)r * s->T + (p % s->T);
}
static int64_t opt_loc(const ora_source* s, int64_t page_id, int64_t p) {
  return (int64_t)s->R * s->B + (int64_t)s->R * s->T + page_id * s->P + (p % s->P);
}
static int64_t stg_loc(const ora_source* s, int32_t r, int64_t c) { return s->stg_base + (int64_t)r * s->S + c; }
static int64_t pool_tag(const ora_source* s, int32_t r, int64_t p) { return (s->uid[r] << 32) | p; }

ora_source* ora_create(int32_t R, const int64_t* ctx, int64_t max_ctx, int32_t B, int32_t T, int32_t page_rows,
                       int64_t opt_pool_pages, int32_t staging_rows, int32_t row_bytes, int64_t stg_base) {
  if (R <= 0 || B <= 0 || T < 0 || page_rows < 0 || opt_pool_pages < 0 || staging_rows < 0) return NULL;
  if (max_ctx <= 0 || max_ctx > 0x7fffffff) return NULL;
  if (page_rows == 0 && opt_pool_pages != 0) return NULL;
  ora_source* s = (ora_source*)calloc(1, sizeof(ora_source));
  if (!s) return NULL;
  s->R = R; s->B = B; s->T = T; s->P = page_rows; s->S = staging_rows; s->row_bytes = row_bytes;
  s->opt_pool_pages = opt_pool_pages;
  s->max_ctx = max_ctx;
  s->ctx = (int64_t*)malloc(sizeof(int64_t) * R);
  s->n_import = (int64_t*)malloc(sizeof(int64_t) * R);
  s->uid = (int64_t*)malloc(sizeof(int64_t) * R);
  s->key = (int32_t*)malloc(sizeof(int32_t) * (size_t)R * B);
  s->rec = (uint32_t*)calloc((size_t)R * B, sizeof(uint32_t));
  s->pt = (int32_t**)calloc(R, sizeof(int32_t*));
  s->opt = (int32_t**)calloc(R, sizeof(int32_t*));
  /* staging follows the optional pages, or sits at stg_base (an arena shared by several sources, [AD] 3.4) */
  const int64_t own = (int64_t)R * B + (int64_t)R * T + opt_pool_pages * page_rows;
  s->stg_base = stg_base >= 0 ? stg_base : own;
  s->pool_rows = own + (int64_t)R * staging_rows;
  if (s->stg_base + (int64_t)R * staging_rows > s->pool_rows) s->pool_rows = s->stg_base + (int64_t)R * staging_rows;
  s->pool = (int64_t*)malloc(sizeof(int64_t) * (size_t)s->pool_rows);
  if (!s->ctx || !s->n_import || !s->uid || !s->key || !s->rec || !s->pt || !s->opt || !s->pool) { ora_destroy(s); return NULL; }
  for (int64_t i = 0; i < s->pool_rows; ++i) s->pool[i] = -1;
  for (int64_t i = 0; i < (int64_t)R * B; ++i) s->key[i] = -1;
  for (int32_t r = 0; r < R; ++r) {
    s->ctx[r] = ctx[r];
    s->n_import[r] = ctx[r];
    s->uid[r] = r;
    if (ctx[r] <= 0 || ctx[r] > max_ctx) { ora_destroy(s); return NULL; }
    s->pt[r] = (int32_t*)malloc(sizeof(int32_t) * (size_t)max_ctx);
    int64_t np = page_rows ? ctx[r] / page_rows : 0;
    s->opt[r] = (int32_t*)malloc(sizeof(int32_t) * (size_t)(np > 0 ? np : 1));
    if (!s->pt[r] || !s->opt[r]) { ora_destroy(s); return NULL; }
    for (int64_t p = 0; p < max_ctx; ++p) s->pt[r][p] = -1;
    for (int64_t g = 0; g < np; ++g) s->opt[r][g] = -1;
  }
  return s;
}

void ora_destroy(ora_source* s) {
  if (!s) return;
  if (s->pt) for (int32_t r = 0; r < s->R; ++r) free(s->pt[r]);
  if (s->opt) for (int32_t r = 0; r < s->R; ++r) free(s->opt[r]);
  free(s->pt); free(s->opt); free(s->ctx); free(s->n_import); free(s->uid); free(s->key); free(s->rec); free(s->pool); free(s);
}

int64_t ora_pool_rows(const ora_source* s) { return s->pool_rows; }

/* [HS] 3.3 (1) and [AD] 3.1: the newest rows stay in the tail, which is never lent. */
void ora_commit_prefill(ora_source* s) {
  for (int32_t r = 0; r < s->R; ++r) {
    int64_t lo = s->ctx[r] - s->T;
    if (lo < 0) lo = 0;
    for (int64_t p = lo; p < s->ctx[r]; ++p) s->pool[tail_loc(s, r, p)] = pool_tag(s, r, p);
  }
}

/* [AD] 3.1 admission: a new request (identity uid) takes slot r with n_rows of imported history.  Its hot
 * cache is reserved empty, it has no optional pages yet, its context is the imported history, and the
 * newest T rows sit in its tail (tail storage is a required allocation, never lent). */
int32_t ora_admit(ora_source* s, int32_t r, int64_t n_rows, int64_t uid) {
  if (r < 0 || r >= s->R || n_rows < 1 || n_rows > s->max_ctx || uid < 0 || uid > 0x7fffffff) return ORA_EINVAL;
  const int64_t np = s->P ? n_rows / s->P : 0;
  int32_t* opt = (int32_t*)malloc(sizeof(int32_t) * (size_t)(np > 0 ? np : 1));
  if (!opt) return ORA_ENOMEM;
  free(s->opt[r]);
  s->opt[r] = opt;
  for (int64_t g = 0; g < np; ++g) s->opt[r][g] = -1;
  for (int32_t j = 0; j < s->B; ++j) {
    s->key[(int64_t)r * s->B + j] = -1;
    s->rec[(int64_t)r * s->B + j] = 0;
  }
  for (int64_t p = 0; p < s->max_ctx; ++p) s->pt[r][p] = -1;
  s->ctx[r] = n_rows;
  s->n_import[r] = n_rows;
  s->uid[r] = uid;
  int64_t lo = n_rows - s->T;
  if (lo < 0) lo = 0;
  for (int64_t p = lo; p < n_rows; ++p) s->pool[tail_loc(s, r, p)] = pool_tag(s, r, p);
  return ORA_OK;
}

/* [AD] 3.1: only whole pages of the history a request brought at admission can be held optionally;
 * populating a page copies it first and then makes its location visible, reclaiming it sets the location
 * back to -1. */
int32_t ora_residency_set(ora_source* s, int32_t r, const int32_t* page_ids, int64_t n_pages) {
  if (r < 0 || r >= s->R || s->P == 0) return ORA_EINVAL;
  int64_t complete = s->n_import[r] / s->P;
  if (n_pages < 0 || n_pages > complete) return ORA_EINVAL;
  for (int64_t g = 0; g < n_pages; ++g)
    if (page_ids[g] < -1 || page_ids[g] >= s->opt_pool_pages) return ORA_EINVAL;
  for (int64_t g = 0; g < n_pages; ++g) {
    s->opt[r][g] = page_ids[g];
    if (page_ids[g] >= 0)
      for (int64_t i = 0; i < s->P; ++i) s->pool[opt_loc(s, page_ids[g], g * s->P + i)] = pool_tag(s, r, g * s->P + i);
  }
  return ORA_OK;
}

/* [HS] 3.3 step 4 and [AD] 3.2: each request's next `count` rows become positions n_r .. n_r + count - 1,
 * produced into the tail (the newest rows are always resident); the rows that leave the tail become
 * history, reachable through the hot cache from their written-through host copies.  Appends are
 * bounded by the reserved rows, and a row stays in the tail across the next append (2 count <= T), the
 * window in which its host copy completes. */
int32_t ora_append(ora_source* s, int32_t count) {
  if (count < 1 || 2 * (int64_t)count > s->T) return ORA_EINVAL;
  for (int32_t r = 0; r < s->R; ++r)
    if (s->ctx[r] + count > s->max_ctx) return ORA_EINVAL;
  for (int32_t r = 0; r < s->R; ++r) {
    for (int32_t i = 0; i < count; ++i) {
      const int64_t p = s->ctx[r] + i;
      s->pool[tail_loc(s, r, p)] = pool_tag(s, r, p);
    }
    s->ctx[r] += count;
  }
  return ORA_OK;
}

int64_t ora_context_rows(const ora_source* s, int32_t r) { return s->ctx[r]; }

/* [AD] Eq. 8: a source packing m token positions per stored row completes, when a request's tokens grow from
 * n to n2, the rows s with floor(n/m) <= s < floor(n2/m) (reading: the upper bound is floored as the lower
 * one, since a row with some of its m positions still missing is not yet complete and remains in the tail). */
int32_t ora_completed_rows(int64_t n, int64_t n2, int32_t m, int64_t* first, int64_t* count) {
  if (m < 1 || n < 0 || n2 < n) return ORA_EINVAL;
  int64_t lo = 0, hi = 0;
  while ((lo + 1) * m <= n) ++lo;      /* floor(n / m), counted out */
  hi = lo;
  while ((hi + 1) * m <= n2) ++hi;     /* floor(n2 / m) */
  *first = lo;
  *count = hi - lo;
  return ORA_OK;
}

/* victim order: ascending (rec, slot) */
typedef struct { uint32_t rec; int32_t slot; } rs_pair;
static int cmp_rs(const void* a, const void* b) {
  const rs_pair* x = (const rs_pair*)a;
  const rs_pair* y = (const rs_pair*)b;
  if (x->rec != y->rec) return x->rec < y->rec ? -1 : 1;
  return x->slot < y->slot ? -1 : (x->slot > y->slot ? 1 : 0);
}

/*
 * One request of one resolve call.  Steps follow [AD] 3.2 / Figure 2 (direct pass, hot-cache scan, host
 * recovery) with the union of [AD] 3.3 Eqs. 5-6, and the hot-cache phases of [HS] 3.4.
 */
static void resolve_request(ora_source* s, int32_t r, uint32_t e, const int32_t* sel, int32_t Qmax, int32_t k,
                            int32_t nq, int32_t* locs, uint8_t* cls, ora_stats* st,
                            int32_t* plan_pos, int32_t* plan_loc, int32_t* plan_n, int32_t plan_cap,
                            int32_t* ev_slot, int32_t* ev_key, int32_t* ev_n) {
  const int64_t n = s->ctx[r];
  const int32_t B = s->B;
  const int64_t nsel = (int64_t)nq * k;
  int32_t* key = s->key + (int64_t)r * B;
  uint32_t* rec = s->rec + (int64_t)r * B;
  int32_t* pt = s->pt[r];
  memset(st, 0, sizeof(*st));
  for (int64_t f = 0; f < (int64_t)Qmax * k; ++f) {
    locs[f] = -1;
    if (cls) cls[f] = ORA_CLS_NONE;
  }
  if (plan_n) plan_n[r] = 0;
  if (ev_n) ev_n[r] = 0;

  /* (1) intake: every selected position must name a row of the request's history ([HS] 3.3 (3)) */
  for (int64_t f = 0; f < nsel; ++f)
    if (sel[f] < 0 || sel[f] >= n) { st->status = ORA_ERANGE; return; }

  /* (2) direct pass, [AD] 3.2 callout 1: tail rows, then ready complete optional pages */
  uint8_t* klass = (uint8_t*)calloc((size_t)(nsel > 0 ? nsel : 1), 1);
  for (int64_t f = 0; f < nsel; ++f) {
    int64_t p = sel[f];
    if (s->T > 0 && p >= n - s->T) {
      klass[f] = ORA_CLS_TAIL;
      locs[f] = (int32_t)tail_loc(s, r, p);
    } else if (s->P > 0 && p / s->P < s->n_import[r] / s->P && s->opt[r][p / s->P] >= 0) {
      /* only complete pages of the imported history are optional ([AD] 3.1); decoded rows are not */
      klass[f] = ORA_CLS_OPT;
      locs[f] = (int32_t)opt_loc(s, s->opt[r][p / s->P], p);
    }
  }

  /* (3) distinct pending positions in first-occurrence order over f = j*k + i ([AD] Eq. 6 union) */
  uint8_t* seen = (uint8_t*)calloc((size_t)n, 1);
  int32_t* uniq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nsel > 0 ? nsel : 1));
  int64_t m = 0;
  for (int64_t f = 0; f < nsel; ++f) {
    if (klass[f] != ORA_CLS_NONE) continue;
    if (!seen[sel[f]]) { seen[sel[f]] = 1; uniq[m++] = sel[f]; }
  }

  /* (4) hot-cache lookup through the page table ([HS] 3.2, 3.4 phases 1-2): hits and misses */
  uint8_t* is_hit_slot = (uint8_t*)calloc((size_t)B, 1);
  int32_t* miss = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
  int64_t nmiss = 0, nhit = 0;
  for (int64_t u = 0; u < m; ++u) {
    int32_t slot = pt[uniq[u]];
    if (slot >= 0) { if (!is_hit_slot[slot]) { is_hit_slot[slot] = 1; ++nhit; } }
    else miss[nmiss++] = uniq[u];
  }

  /* (5) victims ([HS] 3.4 phase 3): non-hit slots by ascending (rec, slot); the first v are taken */
  rs_pair* cand = (rs_pair*)malloc(sizeof(rs_pair) * (size_t)B);
  int32_t ncand = 0;
  for (int32_t slot = 0; slot < B; ++slot)
    if (!is_hit_slot[slot]) { cand[ncand].rec = rec[slot]; cand[ncand].slot = slot; ++ncand; }
  qsort(cand, (size_t)ncand, sizeof(rs_pair), cmp_rs);
  int64_t v = nmiss < ncand ? nmiss : ncand;
  int64_t over = nmiss - v;
  if (over > s->S) {
    st->status = ORA_ESTAGE;
    for (int64_t f = 0; f < (int64_t)Qmax * k; ++f) { locs[f] = -1; if (cls) cls[f] = ORA_CLS_NONE; }
    free(klass); free(seen); free(uniq); free(is_hit_slot); free(miss); free(cand);
    return;
  }

  /* (6) fills: evict the victim's old position, install the missing row, copy host -> pool ([HS] 3.4
   * phases 3-4).  Rows beyond the free slots go to staging ([AD] 3.3), outside the hot cache. */
  int32_t* staged_at = (int32_t*)malloc(sizeof(int32_t) * (size_t)n); /* position -> staging index */
  for (int64_t i = 0; i < nmiss; ++i) staged_at[miss[i]] = -1;
  for (int64_t i = 0; i < nmiss; ++i) {
    int64_t dst;
    if (i < v) {
      int32_t slot = cand[i].slot;
      if (key[slot] >= 0) {
        if (ev_n) {
          ev_slot[(int64_t)r * B + ev_n[r]] = slot;
          ev_key[(int64_t)r * B + ev_n[r]] = key[slot];
          ev_n[r] += 1;
        }
        pt[key[slot]] = -1;
      }
      key[slot] = miss[i];
      pt[miss[i]] = slot;
      rec[slot] = 2u * e;
      dst = hot_loc(s, r, slot);
    } else {
      staged_at[miss[i]] = (int32_t)(i - v);
      dst = stg_loc(s, r, i - v);
    }
    s->pool[dst] = pool_tag(s, r, miss[i]);
    if (plan_n && i < plan_cap) {
      plan_pos[(int64_t)r * plan_cap + i] = miss[i];
      plan_loc[(int64_t)r * plan_cap + i] = (int32_t)dst;
    }
  }
  if (plan_n) plan_n[r] = (int32_t)nmiss;

  /* (7) hits move to the most recent end, above the same step's fills ([HS] 3.2, 3.4 phase 3) */
  for (int32_t slot = 0; slot < B; ++slot)
    if (is_hit_slot[slot]) rec[slot] = 2u * e + 1u;

  /* (8) emit locations in selection order ([HS] 3.4 phase 5; [AD] Eq. 12) */
  uint8_t* missed = seen; /* reuse: 2 = fetched by this call */
  for (int64_t i = 0; i < nmiss; ++i) missed[miss[i]] = 2;
  for (int64_t f = 0; f < nsel; ++f) {
    int64_t p = sel[f];
    if (klass[f] == ORA_CLS_TAIL) { st->n_tail++; }
    else if (klass[f] == ORA_CLS_OPT) { st->n_opt++; }
    else if (missed[p] == 2) {
      st->n_miss_sel++;
      if (staged_at[p] >= 0) { klass[f] = ORA_CLS_STAGED; locs[f] = (int32_t)stg_loc(s, r, staged_at[p]); }
      else { klass[f] = ORA_CLS_FILL; locs[f] = (int32_t)hot_loc(s, r, pt[p]); }
    } else {
      st->n_hit_sel++;
      klass[f] = ORA_CLS_HIT;
      locs[f] = (int32_t)hot_loc(s, r, pt[p]);
    }
    if (cls) cls[f] = klass[f];
  }

  /* (9) stats */
  st->n_sel = (int32_t)nsel;
  st->n_hit = (int32_t)nhit;
  st->n_miss = (int32_t)nmiss;
  st->n_staged = (int32_t)over;
  st->fetched_bytes = nmiss * (int64_t)s->row_bytes;
  st->status = ORA_OK;
  free(klass); free(seen); free(uniq); free(is_hit_slot); free(miss); free(cand); free(staged_at);
}

int32_t ora_resolve(ora_source* s, uint32_t epoch, const int32_t* sel, int32_t Qmax, int32_t k,
                    const int32_t* nq, int32_t* locs, uint8_t* cls, ora_stats* stats,
                    int32_t* plan_pos, int32_t* plan_loc, int32_t* plan_n, int32_t plan_cap,
                    int32_t* ev_slot, int32_t* ev_key, int32_t* ev_n) {
  /* the LRU clock: a caller-supplied epoch, strictly increasing per source */
  if (epoch <= s->last_epoch || epoch > 0x7fffffffu) return ORA_EEPOCH;
  if (Qmax <= 0 || k <= 0) return ORA_EINVAL;
  for (int32_t r = 0; r < s->R; ++r) {
    int32_t q = nq ? nq[r] : Qmax;
    if (q < 0 || q > Qmax) return ORA_EINVAL;
  }
  /* requests are independent (their hot caches, page tables, tails, staging rows and output rows are
   * disjoint), so they may run on several threads; the result does not depend on the thread count */
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < s->R; ++r) {
    int64_t off = (int64_t)r * Qmax * k;
    resolve_request(s, r, epoch, sel + off, Qmax, k, nq ? nq[r] : Qmax, locs + off, cls ? cls + off : NULL,
                    stats + r, plan_pos, plan_loc, plan_n, plan_cap, ev_slot, ev_key, ev_n);
  }
  s->last_epoch = epoch;
  return ORA_OK;
}

/*
 * Promotion copy-back ([AD] 3.4 and Figure 3 callout 3: rows that overflowed into a staging arena; the
 * promoted ones are copied back to stable hot-cache addresses before the arena is released).  The pages do
 * not say which staged rows are promoted; the reading taken here ties promotion to the round's acceptance:
 * queries 0..A_r of request r are committed (the anchor and its A_r accepted drafts, Eq. 7), the others are
 * rejected.  After the resolve at epoch e (the source's last epoch) and the round's attention:
 *   1. P = the distinct staged positions that a committed query selected, in staging order, and that are
 *      not in the hot cache;
 *   2. D = the hot slots touched at epoch e (rec >= 2e) whose position no committed query selected, in
 *      ascending (rec, slot) order: the rows only rejected drafts asked for, fills before hits;
 *   3. for i < min(|P|, |D|): the position held by slot D_i leaves the hot cache, P_i takes the slot with
 *      rec = 2e (a fill of this epoch), and its row is copied from its staging row into the slot's pool row.
 * A second call after the same resolve changes nothing (promoted rows are hot and committed).  locs are the
 * locations that resolve emitted for sel (same layout); accepted[r] is clamped to [0, nq[r] - 1].
 */
int32_t ora_promote(ora_source* s, const int32_t* sel, int32_t Qmax, int32_t k, const int32_t* nq,
                    const int32_t* locs, const int32_t* accepted, int32_t* promoted) {
  if (s->last_epoch == 0 || Qmax <= 0 || k <= 0) return ORA_EINVAL;
  const uint32_t e = s->last_epoch;
  const int32_t B = s->B;
  for (int32_t r = 0; r < s->R; ++r) {
    promoted[r] = 0;
    const int32_t q = nq ? nq[r] : Qmax;
    if (q <= 0) continue;
    int32_t A = accepted[r];
    if (A < 0) A = 0;
    if (A > q - 1) A = q - 1;
    const int32_t* sr = sel + (int64_t)r * Qmax * k;
    const int32_t* lr = locs + (int64_t)r * Qmax * k;
    int32_t* key = s->key + (int64_t)r * B;
    uint32_t* rec = s->rec + (int64_t)r * B;
    int32_t* pt = s->pt[r];
    const int64_t n = s->ctx[r];
    /* committed positions */
    uint8_t* committed = (uint8_t*)calloc((size_t)n, 1);
    for (int32_t j = 0; j <= A; ++j)
      for (int32_t i = 0; i < k; ++i) committed[sr[(int64_t)j * k + i]] = 1;
    /* 1. staged positions selected by a committed query, by staging index, not hot */
    int32_t* pos_at = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s->S > 0 ? s->S : 1));
    for (int32_t c = 0; c < s->S; ++c) pos_at[c] = -1;
    for (int32_t j = 0; j <= A; ++j)
      for (int32_t i = 0; i < k; ++i) {
        const int64_t c = (int64_t)lr[(int64_t)j * k + i] - stg_loc(s, r, 0);
        if (c >= 0 && c < s->S) pos_at[c] = sr[(int64_t)j * k + i];
      }
    int32_t* P = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s->S > 0 ? s->S : 1));
    int32_t* Pc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s->S > 0 ? s->S : 1));
    int32_t np = 0;
    for (int32_t c = 0; c < s->S; ++c)
      if (pos_at[c] >= 0 && pt[pos_at[c]] < 0) { P[np] = pos_at[c]; Pc[np] = c; ++np; }
    /* 2. slots of this epoch holding positions no committed query selected, ascending (rec, slot) */
    rs_pair* D = (rs_pair*)malloc(sizeof(rs_pair) * (size_t)B);
    int32_t nd = 0;
    for (int32_t slot = 0; slot < B; ++slot)
      if (key[slot] >= 0 && rec[slot] >= 2u * e && !committed[key[slot]]) {
        D[nd].rec = rec[slot]; D[nd].slot = slot; ++nd;
      }
    qsort(D, (size_t)nd, sizeof(rs_pair), cmp_rs);
    /* 3. pair and copy back */
    const int32_t m = np < nd ? np : nd;
    for (int32_t i = 0; i < m; ++i) {
      const int32_t slot = D[i].slot;
      pt[key[slot]] = -1;
      key[slot] = P[i];
      pt[P[i]] = slot;
      rec[slot] = 2u * e;
      s->pool[hot_loc(s, r, slot)] = s->pool[stg_loc(s, r, Pc[i])];
    }
    promoted[r] = m;
    free(committed); free(pos_at); free(P); free(Pc); free(D);
  }
  return ORA_OK;
}

void ora_set_threads(int32_t n) {
  if (n > 0) omp_set_num_threads(n);
}

int32_t ora_get_threads(void) { return omp_get_max_threads(); }

void ora_snapshot(const ora_source* s, int32_t r, int32_t* key, uint32_t* rec, int32_t* order, int32_t* pt,
                  int32_t* opt) {
  const int32_t B = s->B;
  if (key) memcpy(key, s->key + (int64_t)r * B, sizeof(int32_t) * (size_t)B);
  if (rec) memcpy(rec, s->rec + (int64_t)r * B, sizeof(uint32_t) * (size_t)B);
  if (order) {
    rs_pair* all = (rs_pair*)malloc(sizeof(rs_pair) * (size_t)B);
    for (int32_t slot = 0; slot < B; ++slot) { all[slot].rec = s->rec[(int64_t)r * B + slot]; all[slot].slot = slot; }
    qsort(all, (size_t)B, sizeof(rs_pair), cmp_rs);
    for (int32_t i = 0; i < B; ++i) order[i] = all[i].slot;
    free(all);
  }
  if (pt) memcpy(pt, s->pt[r], sizeof(int32_t) * (size_t)s->ctx[r]);
  if (opt && s->P > 0) memcpy(opt, s->opt[r], sizeof(int32_t) * (size_t)(s->n_import[r] / s->P));
}

void ora_pool_lookup(const ora_source* s, const int32_t* locs, int64_t n, int64_t* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (locs[i] >= 0 && locs[i] < s->pool_rows) ? s->pool[locs[i]] : -1;
}

/* ---------------------------------------------------------------------------------------------- */
/* attention: the plain definition, [AD] Eq. 1 with exactness of section 3.5                       */
/* ---------------------------------------------------------------------------------------------- */
static double bf16_to_f64(uint16_t h) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)h << 16;
  return (double)v.f;
}

/* softmax(scale * q . k_i) weighted sum of v_i, for one head, from precomputed scores */
static void softmax_weighted(const double* scores, int64_t nk, const uint16_t* vals, int64_t vstride, int32_t dv,
                             double* out) {
  double mx = -INFINITY;
  for (int64_t i = 0; i < nk; ++i) if (scores[i] > mx) mx = scores[i];
  double denom = 0.0;
  for (int32_t c = 0; c < dv; ++c) out[c] = 0.0;
  for (int64_t i = 0; i < nk; ++i) {
    double w = exp(scores[i] - mx);
    denom += w;
    const uint16_t* v = vals + i * vstride;
    for (int32_t c = 0; c < dv; ++c) out[c] += w * bf16_to_f64(v[c]);
  }
  for (int32_t c = 0; c < dv; ++c) out[c] /= denom;
}

void ora_mla_attention(const uint16_t* q, const uint16_t* rows, int32_t k, int32_t H, int32_t dk, int32_t dv,
                       int32_t row_elems, double scale, double* out) {
  double* sc = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  for (int32_t h = 0; h < H; ++h) {
    const uint16_t* qh = q + (int64_t)h * dk;
    for (int32_t i = 0; i < k; ++i) {
      const uint16_t* row = rows + (int64_t)i * row_elems;
      double acc = 0.0;
      for (int32_t d = 0; d < dk; ++d) acc += bf16_to_f64(qh[d]) * bf16_to_f64(row[d]);
      sc[i] = scale * acc;
    }
    softmax_weighted(sc, k, rows, row_elems, dv, out + (int64_t)h * dv);
  }
  free(sc);
}

void ora_gqa_attention(const uint16_t* q, const uint16_t* pages, int32_t kp, int32_t page_tokens, int32_t Hg,
                       int32_t dh, double scale, double* out) {
  const int64_t nk = (int64_t)kp * page_tokens;
  const int64_t tok = 2 * (int64_t)dh; /* one token: [K dh | V dh] */
  double* sc = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  for (int32_t h = 0; h < Hg; ++h) {
    const uint16_t* qh = q + (int64_t)h * dh;
    for (int64_t i = 0; i < nk; ++i) {
      const uint16_t* kv = pages + i * tok;
      double acc = 0.0;
      for (int32_t d = 0; d < dh; ++d) acc += bf16_to_f64(qh[d]) * bf16_to_f64(kv[d]);
      sc[i] = scale * acc;
    }
    softmax_weighted(sc, nk, pages + dh, tok, dh, out + (int64_t)h * dh);
  }
  free(sc);
}

void ora_bf16_from_f64(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    double a = x[i];
    if (a != a) { out[i] = 0x7FC0; continue; }
    /* round the double to 8 significant bits (nearest, ties to even), then take the float bits */
    int ex;
    double m = frexp(fabs(a), &ex);     /* |a| = m * 2^ex, m in [0.5, 1) */
    if (m == 0.0) { out[i] = a < 0 || (a == 0.0 && signbit(a)) ? 0x8000 : 0x0000; continue; }
    double scaled = ldexp(m, 8);        /* 8 significant bits before the point */
    if (ex - 1 < -126) scaled = ldexp(m, 8 - (-126 - (ex - 1)));   /* subnormal range */
    double fl = floor(scaled);
    double frac = scaled - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double mag = (ex - 1 < -126) ? ldexp(fl, -133) : ldexp(fl, ex - 8);
    union { float f; uint32_t u; } v;
    v.f = (float)mag;                   /* exact: mag has at most 8 significant bits */
    if (isinf(v.f) || mag > 3.3895313892515355e38) v.u = 0x7F800000u;
    out[i] = (uint16_t)((v.u >> 16) | (a < 0 ? 0x8000u : 0u));
  }
}

/* [AD] Eq. 4: walk the reclaim order and take the first q requests whose optional pages cover Delta */
int32_t ora_reclaim_plan(const int64_t* pages_held, int32_t n, int64_t deficit) {
  if (deficit <= 0) return 0;
  int64_t acc = 0;
  for (int32_t q = 1; q <= n; ++q) {
    acc += pages_held[q - 1];
    if (acc >= deficit) return q;
  }
  return -1; /* the optional pages do not cover the deficit: admission waits */
}

/* [AD] Eq. 9: R_d = p * ceil((W + p - 1 + K_max) / p) */
int64_t ora_ring_rows(int64_t window, int64_t page_rows, int64_t k_max) {
  int64_t need = window + page_rows - 1 + k_max;
  return page_rows * ((need + page_rows - 1) / page_rows);
}
/* [AD] Eq. 10: phi(i, t) = i * R_d + (t mod R_d) */
int64_t ora_ring_addr(int64_t slot, int64_t t, int64_t ring_rows) { return slot * ring_rows + (t % ring_rows); }
/* [AD] Eq. 11: M_stage = chi * N * K_max * k * d_KV */
double ora_staging_bytes(int64_t live_sources, int64_t slots, int64_t k_max, int64_t k, int64_t row_bytes) {
  return (double)live_sources * (double)slots * (double)k_max * (double)k * (double)row_bytes;
}

/* ---------------------------------------------------------------------------------------------- */
/* cache-policy replay: [HS] 4.3 / Figure 6 (LRU, FIFO, random, Belady on one selection stream)    */
/* ---------------------------------------------------------------------------------------------- */
/* One request's single-query stream sel[steps][k] over positions [0, n) replayed against B slots (B >= k);
 * positions >= tail_from resolve directly and are not cached.  misses[t] = selected positions not resident
 * at step t.  Every policy evicts only slots whose position is not selected in the current step, lowest slot
 * first among equals:
 *   ORA_POLICY_LRU    the deterministic LRU of the hot path (rec = 2e+1 after a hit, 2e after a fill, misses
 *                     take victims in ascending (rec, slot) in first-occurrence order);
 *   ORA_POLICY_FIFO   the earliest filled slot (hits do not refresh);
 *   ORA_POLICY_RANDOM a uniformly random slot (SplitMix64 of seed and a counter);
 *   ORA_POLICY_BELADY the slot whose position is selected again furthest in the future (never: first). */
static uint64_t ora_splitmix(uint64_t* s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int32_t ora_policy_replay(const int32_t* sel, int32_t steps, int32_t k, int64_t n, int64_t tail_from, int32_t B,
                          int32_t policy, uint64_t seed, int32_t* misses) {
  if (steps < 1 || k < 1 || B < k || n < 1 || policy < 0 || policy > 3) return ORA_EINVAL;
  int32_t* slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);   /* position -> slot or -1 */
  int32_t* key = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);       /* slot -> position or -1 */
  int64_t* stamp = (int64_t*)calloc((size_t)B, sizeof(int64_t));      /* LRU rec, FIFO fill order, Belady next use */
  uint8_t* hit = (uint8_t*)calloc((size_t)B, 1);
  int32_t* next_use = (int32_t*)malloc(sizeof(int32_t) * (size_t)steps * k);
  int32_t* last = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  int32_t* pend = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  if (!slot_of || !key || !stamp || !hit || !next_use || !last || !pend) {
    free(slot_of); free(key); free(stamp); free(hit); free(next_use); free(last); free(pend);
    return ORA_ENOMEM;
  }
  for (int64_t p = 0; p < n; ++p) { slot_of[p] = -1; last[p] = 0x7fffffff; }
  for (int32_t b = 0; b < B; ++b) key[b] = -1;
  /* next step at which the position of (t, i) is selected again, from a backward pass */
  for (int32_t t = steps - 1; t >= 0; --t) {
    for (int32_t i = 0; i < k; ++i) next_use[(int64_t)t * k + i] = last[sel[(int64_t)t * k + i]];
    for (int32_t i = 0; i < k; ++i) last[sel[(int64_t)t * k + i]] = t;
  }
  uint64_t rng = seed;
  int64_t fills = 0;
  for (int32_t t = 0; t < steps; ++t) {
    const int32_t* S = sel + (int64_t)t * k;
    const uint32_t e = (uint32_t)t + 1;
    memset(hit, 0, (size_t)B);
    int32_t m = 0;
    /* hits and distinct pending positions in first-occurrence order */
    for (int32_t i = 0; i < k; ++i) {
      const int32_t p = S[i];
      if (p < 0 || p >= n) { m = -1; break; }
      if (p >= tail_from) continue;
      const int32_t sl = slot_of[p];
      if (sl >= 0) {
        hit[sl] = 1;
        if (policy == 0) stamp[sl] = 2 * (int64_t)e + 1;
        if (policy == 3) stamp[sl] = next_use[(int64_t)t * k + i];
      } else {
        int dup = 0;
        for (int32_t j = 0; j < m; ++j) dup |= pend[j] == p;
        if (!dup) pend[m++] = p;
      }
    }
    if (m < 0) { free(slot_of); free(key); free(stamp); free(hit); free(next_use); free(last); free(pend); return ORA_ERANGE; }
    misses[t] = m;
    for (int32_t j = 0; j < m; ++j) {
      /* choose a victim among the slots not hit this step */
      int32_t v = -1;
      if (policy == 2) {
        int32_t cand = 0;
        for (int32_t b = 0; b < B; ++b) cand += !hit[b];
        int64_t pick = (int64_t)(ora_splitmix(&rng) % (uint64_t)cand);
        for (int32_t b = 0; b < B; ++b)
          if (!hit[b] && pick-- == 0) { v = b; break; }
      } else {
        for (int32_t b = 0; b < B; ++b) {
          if (hit[b]) continue;
          if (v < 0) { v = b; continue; }
          if (key[b] < 0 && key[v] >= 0) { v = b; continue; }   /* an empty slot first */
          if ((key[b] < 0) != (key[v] < 0)) continue;
          if (policy == 3 ? stamp[b] > stamp[v] : stamp[b] < stamp[v]) v = b;
        }
      }
      if (key[v] >= 0) slot_of[key[v]] = -1;
      const int32_t p = pend[j];
      key[v] = p;
      slot_of[p] = v;
      hit[v] = 1;   /* a slot filled this step is not a victim again in the same step */
      if (policy == 0) stamp[v] = 2 * (int64_t)e;
      if (policy == 1) stamp[v] = ++fills;
      if (policy == 3) {
        int32_t nu = 0x7fffffff;
        for (int32_t i = 0; i < k; ++i)
          if (S[i] == p) { nu = next_use[(int64_t)t * k + i]; break; }
        stamp[v] = nu;
      }
    }
  }
  free(slot_of); free(key); free(stamp); free(hit); free(next_use); free(last); free(pend);
  return ORA_OK;
}
