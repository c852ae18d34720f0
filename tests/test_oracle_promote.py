"""Pins for the oracle's promotion copy-back (CPU only).

Passage: "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", section 3.4 and
Figure 3 callout 3 (rows that do not fit the hot cache go to a staging arena; promoted rows are copied back to
their stable hot-cache addresses before the arena is reused).  The pages do not say which rows are promoted;
the reading pinned here: after acceptance (Eq. 7) the anchor and the accepted drafts are committed, and staged
rows that a committed query selected take, in staging order, the hot slots that only rejected queries used in
that step, least recently used first.  Checked against an independent brute-force model (explicit recency
list), closed forms and a hand-worked case.
"""
import numpy as np
import pytest

import oracle
from lru_bruteforce import BruteRequest


def _pool_tag(r, p):
    return (int(r) << 32) | int(p)


def _check_state(src, brute, r):
    snap = src.snapshot(r)
    holds = [(-1 if x is None else x) for x in brute.holds]
    assert snap["key"].tolist() == holds
    assert snap["order"].tolist() == brute.recency
    for slot, pos in enumerate(holds):
        if pos >= 0:
            assert snap["pt"][pos] == slot
    assert int((snap["pt"] >= 0).sum()) == sum(1 for x in holds if x >= 0)


def _random_rounds(seed):
    rng = np.random.default_rng(seed)
    R = 3
    B = int(rng.integers(4, 12))
    n = int(rng.integers(B + 8, 60))
    Q = int(rng.integers(2, 5))
    k = int(rng.integers(2, B + 1))
    S = Q * k
    src = oracle.Source(R=R, ctx=n, B=B, T=0, staging_rows=S, row_bytes=16)
    brutes = [BruteRequest(B, n) for _ in range(R)]
    total = 0
    for t in range(8):
        sel = np.zeros((R, Q, k), np.int32)
        for r in range(R):
            for j in range(Q):
                sel[r, j] = rng.choice(n, size=k, replace=False)
        out = src.resolve(t + 1, sel)
        assert out["rc"] == 0
        for r in range(R):
            res = brutes[r].step([list(sel[r, j]) for j in range(Q)], S)
            assert res["error"] is None
            assert list(out["plan"][r][0]) == res["misses"]
        acc = rng.integers(-1, Q + 1, size=R).astype(np.int32)   # out-of-range values are clamped
        got = src.promote(sel, out["locs"], acc)
        for r in range(R):
            pairs = brutes[r].promote([list(sel[r, j]) for j in range(Q)], int(acc[r]))
            assert got[r] == len(pairs)
            _check_state(src, brutes[r], r)
            # the promoted slots hold the staged row's bytes (pool model)
            for slot, pos, _ in pairs:
                assert src.pool_lookup([r * B + slot])[0] == _pool_tag(r, pos)
        total += int(got.sum())
        # a second call after the same resolve changes nothing
        assert src.promote(sel, out["locs"], acc).sum() == 0
    return total


@pytest.mark.parametrize("seed", range(40))
def test_promotion_matches_brute_force_over_random_rounds(seed):
    """Random multi-query rounds that overflow into staging, random acceptance (values outside [0, Q - 1]
    included, clamped): promoted counts, keys, slot order, page table and the promoted rows' bytes agree with
    the brute-force model after every round; a repeated call promotes nothing."""
    _random_rounds(seed)


def test_random_rounds_do_promote_rows():
    assert sum(_random_rounds(seed) for seed in range(40)) > 100


def test_promotion_counts_closed_forms():
    """With every query committed no slot is demotable; with only the anchor committed the count is
    min(|staged rows the anchor selected|, |slots only drafts used|)."""
    R, B, n, Q, k = 1, 6, 40, 3, 6
    rng = np.random.default_rng(7)
    for trial in range(30):
        src = oracle.Source(R=R, ctx=n, B=B, T=0, staging_rows=Q * k, row_bytes=16)
        sel = np.stack([rng.choice(n, size=k, replace=False) for _ in range(Q)])[None].astype(np.int32)
        out = src.resolve(1, sel)
        assert src.promote(sel, out["locs"], [Q - 1])[0] == 0
        src2 = oracle.Source(R=R, ctx=n, B=B, T=0, staging_rows=Q * k, row_bytes=16)
        out2 = src2.resolve(1, sel)
        anchor = set(sel[0, 0].tolist())
        staged = [p for p, l in zip(*out2["plan"][0]) if l >= B]
        snap = src2.snapshot(0)
        only_drafts = [s for s in range(B) if snap["key"][s] >= 0 and snap["key"][s] not in anchor]
        want = min(sum(1 for p in staged if p in anchor), len(only_drafts))
        assert src2.promote(sel, out2["locs"], [0])[0] == want


def test_promotion_hand_worked_example():
    """B = 4 slots, one request.  Epoch 1 resolves one query [33, 34, 35, 36]: slots 0-3 hold them (rec 2).
    Epoch 2 resolves the anchor q0 = [30, 31, 32, 33] and one draft q1 = [34, 35, 36, 37]: the pending rows in
    first-occurrence order are 30 31 32 33 34 35 36 37; 33 34 35 36 hit slots 0-3 (rec 5), so the misses
    30 31 32 37 find no free slot and go to staging rows 0-3.  With the draft rejected (accepted = 0) the
    committed rows are {30, 31, 32, 33}: the staged committed rows are 30 31 32 (rows 0-2); the slots whose row
    only the draft chose are 1 2 3 (34 35 36, all rec 5, ascending slot).  So 30 31 32 move into slots 1 2 3
    as fills of epoch 2 (rec 4), slot 0 stays a hit, the slot order becomes 1 2 3 0, and a next round that
    selects 30 31 32 33 fetches nothing."""
    B, n = 4, 64
    src = oracle.Source(R=1, ctx=n, B=B, T=0, staging_rows=8, row_bytes=16)
    s1 = np.array([[[33, 34, 35, 36]]], np.int32)
    assert src.resolve(1, s1)["rc"] == 0                      # slots 0-3 hold 33 34 35 36 (rec 2)
    s2 = np.array([[[30, 31, 32, 33], [34, 35, 36, 37]]], np.int32)
    out = src.resolve(2, s2)
    # pending in first-occurrence order: 30 31 32 33 34 35 36 37; hits 33 34 35 36 (slots 0-3); misses 30 31 32 37
    # no free slot: all four go to staging rows 0-3
    assert out["plan"][0][0].tolist() == [30, 31, 32, 37]
    assert out["stats"][0]["n_staged"] == 4
    # accepted = 0: committed {30, 31, 32, 33}; staged and committed: 30 31 32 (rows 0 1 2);
    # slots whose row only q1 chose: 34 35 36 in slots 1 2 3 (all hits, rec 5), ascending slot -> 1 2 3
    got = src.promote(s2, out["locs"], [0])
    assert got[0] == 3
    snap = src.snapshot(0)
    assert snap["key"].tolist() == [33, 30, 31, 32]
    assert snap["rec"].tolist() == [5, 4, 4, 4]               # slot 0 stays a hit; 1-3 are fills of epoch 2
    assert snap["order"].tolist() == [1, 2, 3, 0]
    assert snap["pt"][34] == -1 and snap["pt"][30] == 1
    # next round selects 30 31 32 again: all hits now, no host fetch
    out3 = src.resolve(3, np.array([[[30, 31, 32, 33], [30, 31, 32, 33]]], np.int32))
    assert out3["stats"][0]["n_miss"] == 0 and out3["stats"][0]["n_hit"] == 4
