"""Cache-policy replay in the oracle (HiSparse section 4.3, Figure 6): LRU, FIFO, random and Belady on one
request's selection stream, pinned to the resolve oracle, to brute force and to Belady's optimality; plus the
Figure 6 analog on the 100K batch-64 selection stream (printed; recorded with the design notes)."""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _stream(rng, steps, k, n, keep):
    out, prev = [], None
    for _ in range(steps):
        if prev is None:
            cur = rng.choice(n, size=k, replace=False)
        else:
            kept = rng.choice(prev, size=int(keep * k), replace=False)
            pool = np.setdiff1d(np.arange(n), kept)
            cur = np.concatenate([kept, rng.choice(pool, size=k - kept.size, replace=False)])
            rng.shuffle(cur)
        out.append(cur)
        prev = cur
    return np.stack(out).astype(np.int32)


def test_lru_replay_matches_the_resolve_oracle():
    rng = np.random.default_rng(1)
    for B, k, n in ((8, 8, 40), (16, 8, 40), (24, 10, 200), (64, 16, 120)):
        sel = _stream(rng, 25, k, n, 0.6)
        src = oracle.Source(R=1, ctx=n, B=B, T=0, row_bytes=16)
        want = [int(src.resolve(t + 1, sel[t].reshape(1, 1, k))["stats"]["n_miss"][0]) for t in range(sel.shape[0])]
        assert oracle.policy_replay(sel, n, B, "lru").tolist() == want


def _fifo_brute(sel, B):
    """FIFO by an explicit queue of resident positions; victims skip positions selected this step."""
    queue, misses = [], []
    for S in sel:
        sset = set(S.tolist())
        pend = [p for p in dict.fromkeys(S.tolist()) if p not in queue]
        for p in pend:
            if len(queue) >= B:
                victim = next(q for q in queue if q not in sset)
                queue.remove(victim)
            queue.append(p)
        misses.append(len(pend))
    return misses


def test_fifo_replay_matches_brute_force():
    rng = np.random.default_rng(2)
    for B, k, n in ((4, 2, 9), (6, 3, 12), (10, 5, 30), (32, 16, 100)):
        sel = _stream(rng, 30, k, n, 0.5)
        assert oracle.policy_replay(sel, n, B, "fifo").tolist() == _fifo_brute(sel, B)


def _min_misses(sel, B):
    """Exhaustive minimum over every eviction choice (tiny inputs): the offline optimum."""
    best = [None]

    def go(t, cache, acc):
        if best[0] is not None and acc >= best[0]:
            return
        if t == len(sel):
            best[0] = acc
            return
        S = sel[t].tolist()
        pend = [p for p in dict.fromkeys(S) if p not in cache]
        free = B - len(cache)
        evictable = [c for c in cache if c not in S]
        need = max(0, len(pend) - free)
        for ev in itertools.combinations(sorted(evictable), need):
            go(t + 1, (cache - set(ev)) | set(pend), acc + len(pend))
    go(0, frozenset(), 0)
    return best[0]


def test_belady_is_optimal():
    rng = np.random.default_rng(3)
    for _ in range(40):
        B, k, n = int(rng.integers(2, 4)), 1, int(rng.integers(3, 7))
        B = max(B, k)
        sel = rng.integers(0, n, size=(8, k)).astype(np.int32)
        assert int(oracle.policy_replay(sel, n, B, "belady").sum()) == _min_misses(sel, B)
    for _ in range(10):
        sel = _stream(rng, 7, 2, 7, 0.5)
        assert int(oracle.policy_replay(sel, 7, 3, "belady").sum()) == _min_misses(sel, 3)
    # and never worse than the online policies
    for _ in range(10):
        sel = _stream(rng, 40, 16, 300, 0.7)
        bel = int(oracle.policy_replay(sel, 300, 40, "belady").sum())
        for pol in ("lru", "fifo", "random"):
            assert bel <= int(oracle.policy_replay(sel, 300, 40, pol, seed=5).sum())


def test_topk_only_cache_misses_every_new_row():
    """B = k keeps exactly the last selection resident: misses = |S_t minus S_(t-1)| (Figure 6's top-k-only
    staging)."""
    rng = np.random.default_rng(4)
    sel = _stream(rng, 20, 32, 500, 0.7)
    want = [32] + [len(set(sel[t]) - set(sel[t - 1])) for t in range(1, 20)]
    for pol in ("lru", "fifo", "random", "belady"):
        assert oracle.policy_replay(sel, 500, 32, pol, seed=9).tolist() == want


def test_figure6_analog_on_the_100k_stream(capsys):
    """The 100K batch-64 selection stream (80 % kept, Zipf(1.1) fresh rows), first 8 requests of layer 0 over
    32 steps: mean per-step miss rate of each policy and cache size (the pages' Figure 6 used a model trace,
    which is not available; these are the synthetic stand-in's numbers)."""
    w = synth.WORKLOADS["dsa100k"]
    sel = synth.selection_stream(w, 0, steps=32, units=slice(0, 8))   # [steps][8][1][k]
    k = w.top_k
    rows = []
    for name, pol, B in (("top-k only", "lru", k), ("LRU", "lru", 2 * k), ("FIFO", "fifo", 2 * k),
                         ("random", "random", 2 * k), ("Belady", "belady", 2 * k), ("LRU", "lru", 4 * k)):
        m = np.stack([oracle.policy_replay(sel[:, r, 0], w.ctx, B, pol, seed=r) for r in range(8)])
        rate = float(m[:, 1:].sum() / (m.shape[0] * (m.shape[1] - 1) * k))   # steps after the cold first
        rows.append((name, B, rate))
    with capsys.disabled():
        print("\n[policy replay] " + "; ".join(f"{n} B={B}: {100 * r:.1f}%" for n, B, r in rows))
    rate = {(n, B): r for n, B, r in rows}
    assert rate[("Belady", 2 * k)] <= min(rate[("LRU", 2 * k)], rate[("FIFO", 2 * k)], rate[("random", 2 * k)])
    assert rate[("LRU", 4 * k)] <= rate[("LRU", 2 * k)] <= rate[("top-k only", k)]


def _splitmix64(state):
    """SplitMix64 (Vigna's published definition): returns (new state, output)."""
    m = (1 << 64) - 1
    state = (state + 0x9E3779B97F4A7C15) & m
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return state, z ^ (z >> 31)


def test_random_policy_victim_is_uniform_over_non_hit_slots():
    """The random policy's victim is drawn uniformly from the slots not hit in the step: with B slots holding
    a and one other row, re-selecting a after one intervening miss hits unless that miss drew a's slot, so the
    miss frequency over seeds is 1/B; a slot hit in the step is never drawn, so with a hit beside the miss the
    draw is over B - 1 slots.  Binomial bounds at 4 standard deviations over 4,000 seeds."""
    n_seeds = 4000
    n = 100
    a, b, c = 3, 5, 7
    for B in (2, 4):
        sel = np.array([[a], [b], [a]], np.int32)
        miss = np.array([oracle.policy_replay(sel, n, B, "random", seed=s)[2] for s in range(n_seeds)])
        p = 1.0 / B
        assert abs(miss.mean() - p) <= 4 * np.sqrt(p * (1 - p) / n_seeds), (B, miss.mean())
    # B = 3, k = 2: step 1 fills a and b, step 2 hits a and misses c, which draws b's slot or the empty one
    # (1/2 each; a uniform draw over all three slots would give 1/3 and sometimes evict a)
    sel_b = np.array([[a, b], [a, c], [b, b]], np.int32)
    sel_a = np.array([[a, b], [a, c], [a, a]], np.int32)
    miss_b = np.array([oracle.policy_replay(sel_b, n, 3, "random", seed=s)[2] for s in range(n_seeds)])
    miss_a = np.array([oracle.policy_replay(sel_a, n, 3, "random", seed=s)[2] for s in range(n_seeds)])
    assert abs(miss_b.mean() - 0.5) <= 4 * np.sqrt(0.25 / n_seeds), miss_b.mean()
    assert not miss_a.any(), "a slot hit in the step was drawn as a victim"


def test_random_policy_draws_follow_splitmix64():
    """Exact draws: the k-th victim of a stream is output k of SplitMix64 seeded with `seed`, reduced modulo
    the number of candidate slots, counted in slot order.  For [a], [b], [a] with B = 2 the third step misses
    exactly when the first two draws pick the same slot."""
    n, a, b = 50, 11, 12
    sel = np.array([[a], [b], [a]], np.int32)
    for seed in range(64):
        st, r1 = _splitmix64(seed)
        st, r2 = _splitmix64(st)
        want = int(r1 % 2 == r2 % 2)
        got = int(oracle.policy_replay(sel, n, 2, "random", seed=seed)[2])
        assert got == want, seed
