/*
 * Seeded synthetic top-k selection streams, the stand-in for a trained sparse indexer.
 *
 * The pages' selections come from model indexers on real prompts (DSA lightning indexer, NSA block top-k,
 * Quest page bounds); none is available here.  A stream is the ordered list a top-k returns at each decode
 * step, for one (layer or source, request) pair.  Its statistics follow the workload descriptions:
 * a fraction rho of each step's list is kept from the previous step's list, the rest is drawn fresh from
 * a uniform or a Zipf(s) law over positions, without repeating a position inside one list, and the result
 * is shuffled (the order a top-k returns carries no meaning for the cache).
 *
 * This file holds none of the method's arithmetic; it only produces int32 position lists.
 *
 * Random numbers: a SplitMix64 sequence (Steele, Lea and Flood 2014) per stream, seeded by mixing
 * (seed, a, b).  Uniform integers in [0,n) take the high 64 bits of a 128-bit product; a Zipf draw inverts
 * a cumulative table supplied by the caller (smallest index whose cumulative mass exceeds the uniform).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

typedef struct { uint64_t s; } rng_t;

static inline uint64_t rng_next(rng_t* r) { return mix64(r->s += GOLDEN); }
static inline uint32_t rng_below(rng_t* r, uint32_t n) {
  return (uint32_t)(((unsigned __int128)rng_next(r) * n) >> 64);
}
static inline double rng_unit(rng_t* r) { return (double)(rng_next(r) >> 11) * (1.0 / 9007199254740992.0); }

static rng_t rng_for(uint64_t seed, int64_t a, int64_t b) {
  rng_t r;
  uint64_t h = mix64(seed ^ 0x5E1EC7ULL);
  h = mix64(h ^ (GOLDEN * ((uint64_t)a + 0x4000u)));
  h = mix64(h ^ (GOLDEN * ((uint64_t)b + 0x5000u)));
  r.s = h;
  return r;
}

/* one fresh position: uniform over [0,n) (cdf == NULL) or Zipf through the cumulative table cdf[n] */
static inline int32_t draw_pos(rng_t* r, int32_t n, const double* cdf) {
  if (!cdf) return (int32_t)rng_below(r, (uint32_t)n);
  double u = rng_unit(r);
  int32_t lo = 0, hi = n - 1;
  while (lo < hi) {
    int32_t mid = lo + (hi - lo) / 2;
    if (cdf[mid] > u) hi = mid; else lo = mid + 1;
  }
  return lo;
}

/* append `need` fresh positions not yet marked in `taken` (and mark them) */
static void draw_fresh(rng_t* r, int32_t n, const double* cdf, uint8_t* taken, int32_t* dst, int32_t need) {
  int32_t got = 0;
  while (got < need) {
    int32_t p = draw_pos(r, n, cdf);
    if (taken[p]) continue;
    taken[p] = 1;
    dst[got++] = p;
  }
}

/* m entries chosen without replacement from src[len] (partial Fisher-Yates on a scratch copy) */
static void choose(rng_t* r, const int32_t* src, int32_t len, int32_t m, int32_t* dst, int32_t* scratch) {
  memcpy(scratch, src, sizeof(int32_t) * (size_t)len);
  for (int32_t i = 0; i < m; ++i) {
    int32_t j = i + (int32_t)rng_below(r, (uint32_t)(len - i));
    int32_t t = scratch[i]; scratch[i] = scratch[j]; scratch[j] = t;
    dst[i] = scratch[i];
  }
}

static void shuffle(rng_t* r, int32_t* a, int32_t len) {
  for (int32_t i = len - 1; i > 0; --i) {
    int32_t j = (int32_t)rng_below(r, (uint32_t)(i + 1));
    int32_t t = a[i]; a[i] = a[j]; a[j] = t;
  }
}

/*
 * Single-query streams.  out[nb][steps][k] for streams (seed, a, b0 + i), i < nb.
 * Step 0: k distinct fresh positions.  Step t: n_keep chosen from step t-1's list, k - n_keep fresh
 * positions outside the kept ones, then the list is shuffled.
 */
int synth_select_single(int32_t* out, uint64_t seed, int64_t a, int64_t b0, int32_t nb, int32_t steps,
                        int32_t k, int32_t n, int32_t n_keep, const double* cdf, int32_t nthreads) {
  if (k > n || n_keep > k || k <= 0 || steps <= 0 || nb <= 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int32_t i = 0; i < nb; ++i) {
    rng_t r = rng_for(seed, a, b0 + i);
    uint8_t* taken = (uint8_t*)calloc((size_t)n, 1);
    int32_t* scratch = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    if (!taken || !scratch) { bad = 1; free(taken); free(scratch); continue; }
    int32_t* base = out + (int64_t)i * steps * k;
    for (int32_t t = 0; t < steps; ++t) {
      int32_t* cur = base + (int64_t)t * k;
      int32_t kept = 0;
      if (t > 0) {
        choose(&r, cur - k, k, n_keep, cur, scratch);
        kept = n_keep;
        for (int32_t q = 0; q < kept; ++q) taken[cur[q]] = 1;
      }
      draw_fresh(&r, n, cdf, taken, cur + kept, k - kept);
      for (int32_t q = 0; q < k; ++q) taken[cur[q]] = 0;
      shuffle(&r, cur, k);
    }
    free(taken);
    free(scratch);
  }
  return bad ? -2 : 0;
}

/*
 * Multi-query (speculative verification) streams.  out[nb][steps][W][k] for streams (seed, a, b0 + i).
 * Each query's list = a part shared by the request's W queries (n_shared positions) + a private part
 * (k - n_shared).  Each part keeps its own fraction from the previous step (keep_shared, keep_private).
 * Draw order per step: private kept parts (query order), shared kept part, shared fresh part (outside
 * every kept part), then per query its private fresh part (outside the shared part and its own kept
 * part), then per query a shuffle of shared + private.  Private parts of different queries may overlap.
 */
int synth_select_multi(int32_t* out, uint64_t seed, int64_t a, int64_t b0, int32_t nb, int32_t steps,
                       int32_t W, int32_t k, int32_t n, int32_t n_shared, int32_t keep_shared,
                       int32_t keep_private, const double* cdf, int32_t nthreads) {
  const int32_t n_priv = k - n_shared;
  if (k > n || n_shared > k || keep_shared > n_shared || keep_private > n_priv || W <= 0) return -1;
  if ((int64_t)n_shared + (int64_t)W * n_priv > n) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int32_t i = 0; i < nb; ++i) {
    rng_t r = rng_for(seed, a, b0 + i);
    uint8_t* taken = (uint8_t*)calloc((size_t)n, 1);
    int32_t* scratch = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int32_t* shared = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_shared > 0 ? n_shared : 1) * 2);
    int32_t* priv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_priv > 0 ? n_priv : 1) * W * 2);
    if (!taken || !scratch || !shared || !priv) { bad = 1; free(taken); free(scratch); free(shared); free(priv); continue; }
    int32_t* sh_prev = shared; int32_t* sh_cur = shared + n_shared;
    int32_t* pv_prev = priv; int32_t* pv_cur = priv + (int64_t)n_priv * W;
    int32_t* base = out + (int64_t)i * steps * W * k;
    for (int32_t t = 0; t < steps; ++t) {
      int32_t ks = 0, kp = 0;
      if (t > 0) {
        ks = keep_shared; kp = keep_private;
        for (int32_t j = 0; j < W; ++j)
          choose(&r, pv_prev + (int64_t)j * n_priv, n_priv, kp, pv_cur + (int64_t)j * n_priv, scratch);
        choose(&r, sh_prev, n_shared, ks, sh_cur, scratch);
      }
      /* shared fresh: outside the kept shared part and every kept private part */
      for (int32_t q = 0; q < ks; ++q) taken[sh_cur[q]] = 1;
      for (int32_t j = 0; j < W; ++j)
        for (int32_t q = 0; q < kp; ++q) taken[pv_cur[(int64_t)j * n_priv + q]] = 1;
      draw_fresh(&r, n, cdf, taken, sh_cur + ks, n_shared - ks);
      for (int32_t q = 0; q < n_shared; ++q) taken[sh_cur[q]] = 0;
      for (int32_t j = 0; j < W; ++j)
        for (int32_t q = 0; q < kp; ++q) taken[pv_cur[(int64_t)j * n_priv + q]] = 0;
      /* private fresh per query: outside the shared part and that query's kept private part */
      for (int32_t j = 0; j < W; ++j) {
        int32_t* pj = pv_cur + (int64_t)j * n_priv;
        for (int32_t q = 0; q < n_shared; ++q) taken[sh_cur[q]] = 1;
        for (int32_t q = 0; q < kp; ++q) taken[pj[q]] = 1;
        draw_fresh(&r, n, cdf, taken, pj + kp, n_priv - kp);
        for (int32_t q = 0; q < n_shared; ++q) taken[sh_cur[q]] = 0;
        for (int32_t q = 0; q < n_priv; ++q) taken[pj[q]] = 0;
      }
      for (int32_t j = 0; j < W; ++j) {
        int32_t* dst = base + ((int64_t)t * W + j) * k;
        memcpy(dst, sh_cur, sizeof(int32_t) * (size_t)n_shared);
        memcpy(dst + n_shared, pv_cur + (int64_t)j * n_priv, sizeof(int32_t) * (size_t)n_priv);
        shuffle(&r, dst, k);
      }
      int32_t* tmp = sh_prev; sh_prev = sh_cur; sh_cur = tmp;
      tmp = pv_prev; pv_prev = pv_cur; pv_cur = tmp;
    }
    free(taken); free(scratch); free(shared); free(priv);
  }
  return bad ? -2 : 0;
}
