"""Decode-loop append in the oracle (HiSparse section 3.3 step 4; Adaptive DHiSparse section 3.2 and Eq. 8),
pinned to the tail-window arithmetic and to brute force, plus the C ABI's host-side Eq. 8 helper."""
import itertools

import numpy as np
import pytest

import oracle


def _completed_brute(n, n2, m):
    """Rows s complete after the round ((s + 1) m <= n2) that were not complete before ((s + 1) m > n)."""
    rows = [s for s in range(n2 // 1 + 1) if (s + 1) * m <= n2 and (s + 1) * m > n]
    return (rows[0], len(rows)) if rows else None


def test_eq8_completed_rows_brute_force():
    for m in range(1, 6):
        for n in range(0, 23):
            for n2 in range(n, 30):
                got = oracle.completed_rows(n, n2, m)
                want = _completed_brute(n, n2, m)
                if want is None:
                    assert got[1] == 0 and got[0] == n // m, (n, n2, m)
                else:
                    assert got == want, (n, n2, m)
    # m = 1 (no packing): every new position is one completed row
    for n, n2 in itertools.product(range(0, 9), range(0, 12)):
        if n2 >= n:
            assert oracle.completed_rows(n, n2, 1) == (n, n2 - n)
    assert oracle.completed_rows(5, 4, 2) is None and oracle.completed_rows(0, 4, 0) is None


def test_eq8_library_helper_matches_oracle():
    hsk = pytest.importorskip("hierarchical_sparse_kv_layer_amd")
    rng = np.random.default_rng(8)
    for _ in range(2000):
        m = int(rng.integers(1, 64))
        n = int(rng.integers(0, 10 ** 6))
        n2 = n + int(rng.integers(0, 5000))
        assert hsk.completed_rows(n, n2, m) == oracle.completed_rows(n, n2, m)
    with pytest.raises(hsk.HskError):
        hsk.completed_rows(10, 9, 4)


def _sel(positions):
    return np.asarray(positions, np.int32).reshape(1, 1, -1)


def test_append_tail_window_and_history():
    """T = 4, n = 10: the tail is positions 6..9.  Appending 2 rows makes 10, 11 the newest (tail rows
    R*B + r*T + (p mod T)) and moves 6, 7 into history, where a selection misses and fills a hot slot."""
    B, T = 3, 4
    src = oracle.Source(R=1, ctx=10, B=B, T=T, row_bytes=16, max_ctx=20)
    src.commit_prefill()
    o = src.resolve(1, _sel([6, 7, 8, 9]))
    assert o["rc"] == 0 and int(o["stats"]["n_tail"][0]) == 4
    assert o["locs"].reshape(-1).tolist() == [B + p % T for p in (6, 7, 8, 9)]
    assert src.append(2) == 0 and src.context_rows(0) == 12
    o = src.resolve(2, _sel([10, 11, 8, 9, 6, 7]))
    locs = o["locs"].reshape(-1)
    assert locs[:4].tolist() == [B + p % T for p in (10, 11, 8, 9)]
    st = o["stats"][0]
    assert int(st["n_tail"]) == 4 and int(st["n_miss"]) == 2 and int(st["n_hit"]) == 0
    assert o["plan"][0][0].tolist() == [6, 7]                     # the rows that left the tail, in miss order
    assert set(locs[4:].tolist()) <= set(range(B))                # filled into hot slots
    # the pool model: every emitted location holds the selected row (Eq. 12)
    tags = src.pool_lookup(locs)
    assert tags.tolist() == [p for p in (10, 11, 8, 9, 6, 7)]
    # the new rows occupy the ring slots of the rows they replaced
    assert src.pool_lookup(np.array([B + 10 % T, B + 11 % T], np.int32)).tolist() == [10, 11]


def test_append_rejections_change_nothing():
    src = oracle.Source(R=2, ctx=[10, 17], B=4, T=6, row_bytes=16, max_ctx=20)
    src.commit_prefill()
    assert src.append(4) == oracle.EINVAL                   # 2 count > T
    assert src.append(0) == oracle.EINVAL
    assert src.append(3) == 0                                     # 13, 20
    assert src.append(1) == oracle.EINVAL                   # request 1 would pass max_ctx
    assert [src.context_rows(r) for r in range(2)] == [13, 20]
    # positions at or beyond the context stay out of range
    o = src.resolve(1, np.array([[[12, 13]], [[19, 5]]], np.int32))
    assert int(o["stats"]["status"][0]) == oracle.ERANGE and int(o["stats"]["status"][1]) == 0


def test_append_keeps_optional_pages_to_the_imported_history():
    """Rows generated during decoding stay under the tail and hot-cache rules (Adaptive DHiSparse 3.1): the
    optional map only covers complete pages of the imported history."""
    src = oracle.Source(R=1, ctx=32, B=4, T=4, page_rows=8, opt_pool_pages=8, row_bytes=16, max_ctx=64)
    src.commit_prefill()
    for _ in range(8):
        assert src.append(2) == 0
    assert src.context_rows(0) == 48
    assert src.residency_set(0, [0, 1, 2, 3]) == 0
    assert src.residency_set(0, [0, 1, 2, 3, 4]) == oracle.EINVAL
    # a decoded row outside the tail is fetched into the hot cache, never read from the optional pool
    o = src.resolve(1, _sel([40, 3]))
    st = o["stats"][0]
    assert int(st["n_opt"]) == 1 and int(st["n_miss"]) == 1 and o["plan"][0][0].tolist() == [40]


def test_append_many_steps_matches_brute_force_tail():
    """Random appends and selections: a selection is direct from the tail exactly when p >= n_r - T, and
    every emitted location holds the selected row."""
    rng = np.random.default_rng(3)
    R, B, T, k = 3, 16, 8, 12
    ctx = np.array([40, 9, 100], np.int64)
    src = oracle.Source(R=R, ctx=ctx, B=B, T=T, row_bytes=16, max_ctx=200)
    src.commit_prefill()
    n = ctx.copy()
    for e in range(1, 30):
        c = int(rng.integers(1, T // 2 + 1))
        assert src.append(c) == 0
        n += c
        sel = np.stack([rng.choice(int(n[r]), size=k, replace=False) for r in range(R)]).astype(np.int32)[:, None]
        o = src.resolve(e, sel)
        assert o["rc"] == 0
        for r in range(R):
            tail = sel[r, 0] >= n[r] - T
            assert int(o["stats"]["n_tail"][r]) == int(tail.sum())
            locs = o["locs"][r, 0]
            assert np.array_equal(locs[tail], R * B + r * T + sel[r, 0][tail] % T)
            tags = src.pool_lookup(locs)
            assert np.array_equal(tags, (r << 32) | sel[r, 0].astype(np.int64))


def test_ring_rows_library_helper_matches_oracle():
    """Adaptive DHiSparse Eq. 9 in the C ABI (host function) against the oracle and the worked example."""
    hsk = pytest.importorskip("hierarchical_sparse_kv_layer_amd")
    assert hsk.ring_rows(2048, 64, 8) == 2176
    for window, p, k_max in itertools.product((1, 7, 64, 1000, 2048, 4097), (1, 2, 16, 64), (1, 4, 8, 16)):
        assert hsk.ring_rows(window, p, k_max) == oracle.ring_rows(window, p, k_max)
    with pytest.raises(hsk.HskError):
        hsk.ring_rows(0, 64, 8)
