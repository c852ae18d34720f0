"""Pins for the oracle's resolver: brute force, closed forms, invariants (CPU only).

Passages: HiSparse section 3.2 (hot cache of B >= k slots, page table, LRU with hits promoted above the
same step's fills), section 3.4 (resolve phases); Adaptive DHiSparse section 3.2 / Figure 2 (direct pass
before the hot scan), section 3.3 Eqs. 5-6 (union, each distinct missing row fetched once, staging),
section 3.5 Eq. 12 (every emitted location holds the selected row).
"""
import itertools

import numpy as np
import pytest

import oracle
from lru_bruteforce import BruteRequest

CLS_NAME = {oracle.CLS_TAIL: "tail", oracle.CLS_OPT: "opt", oracle.CLS_HIT: "hit", oracle.CLS_FILL: "fill",
            oracle.CLS_STAGED: "staged"}


def _compare_step(src, brute, r, out, lists, k):
    """Oracle result of request r against the brute-force model's step result."""
    b = brute
    cls = [CLS_NAME[c] for j in range(len(lists)) for c in out["cls"][r, j, :k]]
    assert cls == b["classes"]
    pos, loc = out["plan"][r]
    assert list(pos) == b["misses"]
    B = src.B
    hot_fills = [int(l) - r * B for l in loc[:len(b["victims"])]]
    assert hot_fills == b["victims"]
    ev_slot, ev_key = out["evictions"][r]
    assert list(zip(ev_slot.tolist(), ev_key.tolist())) == b["evictions"]
    st = out["stats"][r]
    assert st["n_hit"] == len(b["hit_slots"])
    assert st["n_miss"] == len(b["misses"])
    assert st["n_staged"] == len(b["staged"])


def _run_pair(R, n, B, T, k, Q, steps, rng, page_rows=0, ready=None, staging=0, distinct=True):
    src = oracle.Source(R=R, ctx=n, B=B, T=T, page_rows=page_rows, opt_pool_pages=(n // page_rows) * R if page_rows else 0,
                        staging_rows=staging, row_bytes=16)
    src.commit_prefill()
    brutes = [BruteRequest(B, n, T, page_rows) for _ in range(R)]
    if page_rows and ready is not None:
        for r in range(R):
            ids = [-1] * (n // page_rows)
            for g in ready[r]:
                ids[g] = r * (n // page_rows) + g
                brutes[r].ready_pages[g] = ids[g]
            assert src.residency_set(r, ids) == 0
    for t in range(steps):
        sel = np.zeros((R, Q, k), np.int32)
        for r in range(R):
            for j in range(Q):
                if distinct:
                    sel[r, j] = rng.choice(n, size=k, replace=False)
                else:
                    sel[r, j] = rng.integers(0, n, size=k)
        out = src.resolve(t + 1, sel)
        assert out["rc"] == 0
        for r in range(R):
            b = brutes[r].step([list(sel[r, j]) for j in range(Q)], staging)
            if b["error"]:
                assert out["stats"][r]["status"] == oracle.ESTAGE
                continue
            assert out["stats"][r]["status"] == 0
            _compare_step(src, b, r, out, [sel[r, j] for j in range(Q)], k)
            snap = src.snapshot(r)
            assert list(snap["order"]) == brutes[r].recency
            assert [(-1 if p is None else p) for p in brutes[r].holds] == list(snap["key"])
        # Eq. 12 through the pool model
        tags = src.pool_lookup(out["locs"])
        ok = np.array([out["stats"][r]["status"] == 0 for r in range(R)])
        want = (np.arange(R, dtype=np.int64)[:, None, None] << 32) | sel.astype(np.int64)
        assert np.array_equal(tags[ok], want[ok])
    return src


def test_exhaustive_tiny_single_query():
    """Every ordered 2-of-4 selection sequence of 4 steps, B=2 (HiSparse 3.2: B >= k)."""
    lists = list(itertools.permutations(range(4), 2))
    for seq in itertools.product(lists, repeat=3):
        src = oracle.Source(R=1, ctx=4, B=2, T=0, row_bytes=16)
        br = BruteRequest(2, 4)
        for t, lst in enumerate(seq):
            out = src.resolve(t + 1, np.array([[lst]], np.int32))
            b = br.step([list(lst)], 0)
            _compare_step(src, b, 0, out, [np.array(lst)], 2)
            assert list(src.snapshot(0)["order"]) == br.recency


def test_exhaustive_tiny_two_queries_with_staging():
    """Two queries of 2 over 5 positions, B=2, staging 2: unions overflow into staging."""
    lists = list(itertools.permutations(range(5), 2))
    rng = np.random.default_rng(5)
    for _ in range(400):
        seq = [(lists[rng.integers(len(lists))], lists[rng.integers(len(lists))]) for _ in range(4)]
        src = oracle.Source(R=1, ctx=5, B=2, T=0, staging_rows=2, row_bytes=16)
        br = BruteRequest(2, 5)
        for t, (a, b_) in enumerate(seq):
            out = src.resolve(t + 1, np.array([[a, b_]], np.int32))
            b = br.step([list(a), list(b_)], 2)
            _compare_step(src, b, 0, out, [np.array(a), np.array(b_)], 2)
            assert list(src.snapshot(0)["order"]) == br.recency


@pytest.mark.parametrize("case", range(40))
def test_random_small_against_bruteforce(case):
    rng = np.random.default_rng(1000 + case)
    n = int(rng.integers(8, 60))
    B = int(rng.integers(1, 12))
    k = int(rng.integers(1, min(B, n) + 1))
    T = int(rng.integers(0, 4))
    Q = int(rng.integers(1, 4))
    page_rows = int(rng.choice([0, 4]))
    ready = None
    if page_rows:
        ready = [set(rng.choice(n // page_rows, size=int(rng.integers(0, n // page_rows + 1)), replace=False).tolist())
                 for _ in range(3)]
    staging = int(rng.integers(0, Q * k + 1))
    _run_pair(R=3, n=n, B=B, T=T, k=k, Q=Q, steps=6, rng=rng, page_rows=page_rows, ready=ready, staging=staging,
              distinct=bool(case % 3))


def test_closed_form_B_equals_k():
    """B = k with no tail or optional pages keeps exactly the current top-k (HiSparse 4.3, top-k-only
    staging): misses at step t+1 = |S_{t+1} \\ S_t|."""
    rng = np.random.default_rng(7)
    n, k = 200, 16
    src = oracle.Source(R=1, ctx=n, B=k, T=0, row_bytes=16)
    prev = None
    for t in range(30):
        lst = rng.choice(n, size=k, replace=False) if prev is None or t % 5 == 0 else \
            np.concatenate([rng.choice(prev, size=10, replace=False),
                            rng.choice(np.setdiff1d(np.arange(n), prev), size=6, replace=False)])
        out = src.resolve(t + 1, lst.reshape(1, 1, k).astype(np.int32))
        want = k if prev is None else len(set(lst) - set(prev))
        assert out["stats"][0]["n_miss"] == want
        assert set(src.snapshot(0)["key"]) == set(lst)
        prev = lst


def test_closed_form_B_at_least_n():
    """B >= n: a row misses only on its first selection."""
    rng = np.random.default_rng(8)
    n, k = 40, 7
    src = oracle.Source(R=1, ctx=n, B=n, T=0, row_bytes=16)
    touched = set()
    for t in range(25):
        lst = rng.choice(n, size=k, replace=False)
        out = src.resolve(t + 1, lst.reshape(1, 1, k).astype(np.int32))
        assert out["stats"][0]["n_miss"] == len(set(lst) - touched)
        assert out["evictions"][0][0].size == 0
        touched |= set(lst.tolist())


def test_lru_inclusion_and_no_self_eviction():
    """Single query, B >= k: (a) no victim holds a row selected in the same call (HiSparse 3.2: B >= k
    so the current selection always fits); (b) every cached row was last selected no earlier than any
    row that was selected before and is not cached (LRU inclusion)."""
    rng = np.random.default_rng(9)
    n, B, k = 120, 24, 10
    src = oracle.Source(R=1, ctx=n, B=B, T=0, row_bytes=16)
    last = {}
    prev = rng.choice(n, size=k, replace=False)
    for t in range(60):
        keep = rng.choice(prev, size=6, replace=False)
        fresh = rng.choice(np.setdiff1d(np.arange(n), keep), size=k - 6, replace=False)
        lst = rng.permutation(np.concatenate([keep, fresh]))
        out = src.resolve(t + 1, lst.reshape(1, 1, k).astype(np.int32))
        ev_slot, ev_key = out["evictions"][0]
        assert not (set(ev_key.tolist()) & set(lst.tolist()))
        for p in lst:
            last[int(p)] = t + 1
        cached = set(int(p) for p in src.snapshot(0)["key"] if p >= 0)
        assert set(lst.tolist()) <= cached
        outside = [last[p] for p in last if p not in cached]
        if outside:
            assert min(last[p] for p in cached) >= max(outside)
        prev = lst


def test_page_table_key_bijection_and_conservation():
    rng = np.random.default_rng(10)
    R, n, B, T, k, Q = 2, 300, 32, 8, 12, 3
    src = oracle.Source(R=R, ctx=n, B=B, T=T, page_rows=16, opt_pool_pages=40, staging_rows=Q * k, row_bytes=16)
    src.commit_prefill()
    ids = [-1] * (n // 16)
    for g in (0, 3, 5, 17):
        ids[g] = g
    assert src.residency_set(0, ids) == 0
    for t in range(20):
        sel = rng.integers(0, n, size=(R, Q, k)).astype(np.int32)
        out = src.resolve(t + 1, sel)
        for r in range(R):
            st = out["stats"][r]
            assert st["n_tail"] + st["n_opt"] + st["n_hit_sel"] + st["n_miss_sel"] == st["n_sel"] == Q * k
            # direct-pass closed forms
            flat = sel[r].reshape(-1)
            assert st["n_tail"] == int(np.sum(flat >= n - T))
            if r == 0:
                ready = {g for g, v in enumerate(ids) if v >= 0}
                assert st["n_opt"] == int(sum(1 for p in flat if p < n - T and p // 16 in ready))
            else:
                assert st["n_opt"] == 0
            assert st["fetched_bytes"] == st["n_miss"] * 16
            snap = src.snapshot(r)
            for s_, p in enumerate(snap["key"]):
                if p >= 0:
                    assert snap["pt"][p] == s_
            assert int(np.sum(snap["pt"] >= 0)) == int(np.sum(snap["key"] >= 0))
            # staged count: misses beyond the free (non-hit) slots
            assert st["n_staged"] == max(0, st["n_miss"] - (B - st["n_hit"]))


def test_errors_leave_request_unchanged():
    src = oracle.Source(R=2, ctx=[50, 50], B=4, T=2, staging_rows=1, row_bytes=16)
    src.commit_prefill()
    out = src.resolve(1, np.array([[[1, 2, 3]], [[4, 5, 6]]], np.int32))
    before = [src.snapshot(r) for r in range(2)]
    # out-of-range position in request 0 only
    out = src.resolve(2, np.array([[[1, 2, 50]], [[7, 8, 9]]], np.int32))
    assert out["stats"][0]["status"] == oracle.ERANGE and out["stats"][1]["status"] == 0
    assert np.all(out["locs"][0] == -1)
    a = src.snapshot(0)
    for key in ("key", "rec", "pt"):
        assert np.array_equal(a[key], before[0][key])
    # negative position
    out = src.resolve(3, np.array([[[-1, 2, 3]], [[7, 8, 9]]], np.int32))
    assert out["stats"][0]["status"] == oracle.ERANGE
    # staging overflow: 2 queries of 3 distinct new rows -> 6 misses, 4 slots, 1 staging row
    before = src.snapshot(1)
    out = src.resolve(4, np.array([[[1, 2, 3], [1, 2, 3]], [[20, 21, 22], [23, 24, 25]]], np.int32))
    assert out["stats"][1]["status"] == oracle.ESTAGE
    a = src.snapshot(1)
    for key in ("key", "rec", "pt"):
        assert np.array_equal(a[key], before[key])
    # epoch must increase
    assert src.resolve(4, np.array([[[1, 2, 3]], [[4, 5, 6]]], np.int32))["rc"] == oracle.EEPOCH
    assert src.resolve(3, np.array([[[1, 2, 3]], [[4, 5, 6]]], np.int32))["rc"] == oracle.EEPOCH


def test_multiquery_dedup_identical_and_disjoint():
    """Adaptive DHiSparse 3.3 / Figure 8a caption: identical queries fetch one payload, disjoint queries
    fetch one payload each."""
    n, k, W, B = 5000, 64, 8, 128
    rng = np.random.default_rng(11)
    base = rng.choice(n, size=k, replace=False)
    src = oracle.Source(R=1, ctx=n, B=B, T=0, staging_rows=W * k, row_bytes=576)
    one = src.resolve(1, base.reshape(1, 1, k).astype(np.int32))["stats"][0]["fetched_bytes"]
    src = oracle.Source(R=1, ctx=n, B=B, T=0, staging_rows=W * k, row_bytes=576)
    same = src.resolve(1, np.tile(base, (1, W, 1)).astype(np.int32))["stats"][0]
    assert same["fetched_bytes"] == one == k * 576
    assert same["n_miss_sel"] == W * k
    dis = rng.choice(n, size=W * k, replace=False).reshape(1, W, k).astype(np.int32)
    src = oracle.Source(R=1, ctx=n, B=B, T=0, staging_rows=W * k, row_bytes=576)
    st = src.resolve(1, dis)["stats"][0]
    assert st["fetched_bytes"] == W * one
    assert st["n_staged"] == W * k - B


def test_dedup_ratio_and_saved_fraction():
    """1.41 missing selections per distinct fetched row removes 1 - 1/1.41 = 29% of fetches
    (Adaptive DHiSparse 4.3.2)."""
    rng = np.random.default_rng(12)
    n, k, W = 3000, 40, 4
    src = oracle.Source(R=1, ctx=n, B=4 * k, T=0, staging_rows=W * k, row_bytes=16)
    shared = rng.choice(n, size=k // 2, replace=False)
    lists = [np.concatenate([shared, rng.choice(np.setdiff1d(np.arange(n), shared), size=k - k // 2, replace=False)])
             for _ in range(W)]
    st = src.resolve(1, np.array([lists], np.int32))["stats"][0]
    rho = st["n_miss_sel"] / st["n_miss"]
    saved = 1.0 - st["n_miss"] / st["n_miss_sel"]
    assert abs(saved - (1 - 1 / rho)) < 1e-12
    assert abs((1 - 1 / 1.41) - 0.29) < 0.005


def test_resolve_does_not_depend_on_thread_count():
    """The request-parallel loop of the oracle resolve gives the same locations, stats, plans and states on
    one thread and on several."""
    rng = np.random.default_rng(123)
    R, n, B, T, Q, k = 16, 400, 32, 8, 3, 24
    sels = [np.stack([np.stack([rng.choice(n, size=k, replace=False) for _ in range(Q)]) for _ in range(R)])
            .astype(np.int32) for _ in range(5)]
    outs = []
    for threads in (1, 7):
        oracle.set_threads(threads)
        src = oracle.Source(R=R, ctx=n, B=B, T=T, staging_rows=Q * k, row_bytes=16)
        src.commit_prefill()
        res = [src.resolve(t + 1, sels[t]) for t in range(5)]
        outs.append((res, [src.snapshot(r) for r in range(R)]))
    oracle.set_threads(0)
    (a, sa), (b, sb) = outs
    for x, y in zip(a, b):
        assert np.array_equal(x["locs"], y["locs"]) and np.array_equal(x["stats"], y["stats"])
        for (p1, l1), (p2, l2) in zip(x["plan"], y["plan"]):
            assert np.array_equal(p1, p2) and np.array_equal(l1, l2)
    for x, y in zip(sa, sb):
        for f in ("key", "rec", "order", "pt"):
            assert np.array_equal(x[f], y[f])
