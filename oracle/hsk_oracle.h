/*
 * CPU oracle of the hierarchical sparse KV hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke entry point and the benchmark's CPU-baseline leg may load or call this
 * library.  The HIP product path never links, includes or calls it, and it shares no code with it.
 *
 * What it computes (plain, slow, step by step):
 *   - ora_resolve: the residency-aware resolver of "Adaptive DHiSparse: Speculative Decoding over a
 *     Load-Adaptive KV Hierarchy" (section 3.2 and Figure 2: tail and ready optional history first, then
 *     the bounded hot cache, then host recovery into the hot cache; section 3.3 Eqs. 5-6: the union of a
 *     request's queries with each distinct missing row fetched once, overflow rows to staging), over the
 *     LRU hot cache of "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV Cache
 *     Management" (section 3.2: page table, B >= k, hits promoted above same-step fills; section 3.4
 *     phases 1-5).  LRU ties are broken by the lowest slot index.
 *   - ora_mla_attention / ora_gqa_attention: the plain definition of softmax attention over the selected
 *     rows in fp64 (Adaptive DHiSparse Eq. 1; exactness in section 3.5).
 *   - ora_reclaim_plan: the whole-request reclaim rule, Adaptive DHiSparse Eq. 4.
 *   - a pool model (which host row each pool row holds) so that Eq. 12 of Adaptive DHiSparse,
 *     KV[loc] = c_{r,s}, can be checked for every emitted location.
 *   - ora_promote: promotion copy-back of staged rows after the round's acceptance (section 3.4).
 *   - sizing closed forms: the draft ring (Eq. 9), ring address (Eq. 10), staging reservation (Eq. 11).
 */
#ifndef HSK_ORACLE_H
#define HSK_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORA_OK = 0, ORA_EINVAL = -1, ORA_ENOMEM = -2, ORA_ERANGE = -5, ORA_ESTAGE = -6, ORA_EEPOCH = -7 };

/* per-selection class codes */
enum { ORA_CLS_NONE = 0, ORA_CLS_TAIL = 1, ORA_CLS_OPT = 2, ORA_CLS_HIT = 3, ORA_CLS_FILL = 4, ORA_CLS_STAGED = 5 };

typedef struct {
  int32_t n_sel;       /* selections examined (sum of query list lengths) */
  int32_t n_tail;      /* selections resolved from the tail */
  int32_t n_opt;       /* selections resolved from ready optional-history pages */
  int32_t n_hit;       /* distinct hot-cache hit slots */
  int32_t n_hit_sel;   /* selections resolved by hot-cache hits */
  int32_t n_miss;      /* distinct missing rows fetched from host (hot fills + staged) */
  int32_t n_miss_sel;  /* selections resolved by this call's fetches */
  int32_t n_staged;    /* distinct missing rows placed in staging */
  int32_t status;      /* ORA_OK / ORA_ERANGE / ORA_ESTAGE */
  int32_t pad;
  int64_t fetched_bytes;
} ora_stats;

typedef struct ora_source ora_source;

/* One payload source: R requests, each with B hot slots, T tail rows, an optional-history page map over
 * its complete pages, and staging_rows staging rows; opt_pool_pages optional pages shared by the source.
 * Pool row layout: [R*B hot][R*T tail][opt_pool_pages*page_rows optional][R*staging_rows staging]. */
ora_source* ora_create(int32_t R, const int64_t* ctx, int64_t max_ctx, int32_t B, int32_t T, int32_t page_rows,
                       int64_t opt_pool_pages, int32_t staging_rows, int32_t row_bytes, int64_t stg_base);
void ora_destroy(ora_source* s);
int64_t ora_pool_rows(const ora_source* s);

/* tail rows are written by prefill and stay resident */
void ora_commit_prefill(ora_source* s);
/* map entries for complete pages [0, n_pages) of request r: page id in the optional pool, or -1 */
int32_t ora_residency_set(ora_source* s, int32_t r, const int32_t* page_ids, int64_t n_pages);
int32_t ora_append(ora_source* s, int32_t count);
/* a new request (identity uid, n_rows of imported history) takes slot r: empty hot cache, no optional pages,
 * its newest T rows in the tail; pool rows are tagged with uid from then on */
int32_t ora_admit(ora_source* s, int32_t r, int64_t n_rows, int64_t uid);
int64_t ora_context_rows(const ora_source* s, int32_t r);
int32_t ora_completed_rows(int64_t n, int64_t n2, int32_t m, int64_t* first, int64_t* count);

/* One resolve call over sel[R][Qmax][k] (query j of request r uses its first k entries when j < nq[r]).
 * Outputs (all may be NULL except locs and stats):
 *   locs[R][Qmax][k]  pool row of every selection (-1 where not produced)
 *   cls[R][Qmax][k]   class code of every selection
 *   stats[R]
 *   plan_pos[R][plan_cap], plan_loc[R][plan_cap], plan_n[R]: distinct missing rows in miss order and
 *     the pool row each was copied to
 *   ev_slot[R][B], ev_key[R][B], ev_n[R]: evictions (slot, position it held) in victim order
 * Returns ORA_EEPOCH (nothing changed) when epoch <= the last accepted epoch, else ORA_OK. */
int32_t ora_resolve(ora_source* s, uint32_t epoch, const int32_t* sel, int32_t Qmax, int32_t k,
                    const int32_t* nq, int32_t* locs, uint8_t* cls, ora_stats* stats,
                    int32_t* plan_pos, int32_t* plan_loc, int32_t* plan_n, int32_t plan_cap,
                    int32_t* ev_slot, int32_t* ev_key, int32_t* ev_n);

/* Promotion copy-back after the last resolve ([AD] 3.4, Figure 3 callout 3), read as: queries 0..accepted[r]
 * of request r are committed; staged rows that a committed query selected take, in staging order, the hot
 * slots of this epoch whose rows only rejected queries selected, in ascending (rec, slot) order, and are copied
 * there from staging.  sel and locs: the last resolve's selections and emitted locations.  promoted[R] out. */
int32_t ora_promote(ora_source* s, const int32_t* sel, int32_t Qmax, int32_t k, const int32_t* nq,
                    const int32_t* locs, const int32_t* accepted, int32_t* promoted);

/* threads of the request-parallel loop in ora_resolve (OpenMP); results do not depend on it */
void ora_set_threads(int32_t n);
int32_t ora_get_threads(void);

/* state of request r: key[B], rec[B], order[B] (slots ascending by (rec, slot)), pt[ctx_r], opt[pages_r] */
void ora_snapshot(const ora_source* s, int32_t r, int32_t* key, uint32_t* rec, int32_t* order, int32_t* pt,
                  int32_t* opt);
/* pool model lookup: out[i] = r * 2^32 + position held by pool row locs[i], or -1 */
void ora_pool_lookup(const ora_source* s, const int32_t* locs, int64_t n, int64_t* out);

/* fp64 softmax attention over k selected rows (bf16 bit patterns):
 * q[H][dk], rows[k][row_elems]; keys = row[0:dk], values = row[0:dv]; out[H][dv] */
void ora_mla_attention(const uint16_t* q, const uint16_t* rows, int32_t k, int32_t H, int32_t dk, int32_t dv,
                       int32_t row_elems, double scale, double* out);
/* GQA over kp selected pages of page_tokens tokens, each token [K dh | V dh]; q[Hg][dh]; out[Hg][dh] */
void ora_gqa_attention(const uint16_t* q, const uint16_t* pages, int32_t kp, int32_t page_tokens, int32_t Hg,
                       int32_t dh, double scale, double* out);
/* fp64 -> bf16, round to nearest even */
void ora_bf16_from_f64(const double* x, uint16_t* out, int64_t n);

/* Eq. 4: smallest q with a_1 + ... + a_q >= deficit over the reclaim order; -1 if no q covers it */
int32_t ora_reclaim_plan(const int64_t* pages_held, int32_t n, int64_t deficit);

/* Eq. 9 draft ring rows, Eq. 10 ring address, Eq. 11 staging reservation (bytes) */
int64_t ora_ring_rows(int64_t window, int64_t page_rows, int64_t k_max);
int64_t ora_ring_addr(int64_t slot, int64_t t, int64_t ring_rows);
double ora_staging_bytes(int64_t live_sources, int64_t slots, int64_t k_max, int64_t k, int64_t row_bytes);

/* [HS] 4.3 / Figure 6: replacement policies replayed on one single-query selection stream (test use) */
enum { ORA_POLICY_LRU = 0, ORA_POLICY_FIFO = 1, ORA_POLICY_RANDOM = 2, ORA_POLICY_BELADY = 3 };
int32_t ora_policy_replay(const int32_t* sel, int32_t steps, int32_t k, int64_t n, int64_t tail_from, int32_t B,
                          int32_t policy, uint64_t seed, int32_t* misses);

#ifdef __cplusplus
}
#endif
#endif
