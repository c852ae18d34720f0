"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Indexing (locations, hit/miss sets, victims via the plan and slot order, page tables, fetched bytes) must
be bit-exact; attention within |gpu - ref| <= 1e-2 + 2e-2 |ref| of the fp64 oracle (bf16 outputs).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_sparse_kv_layer_amd as hsk  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from hsk_harness import Harness, log, ATOL, RTOL  # noqa: E402


def test_tiny_every_step_every_query():
    """Small MLA decode: 4 requests, 8 steps; every location, plan, metadata, pool byte and attention
    output checked."""
    h = Harness(synth.WORKLOADS["tiny"])
    for t in range(h.steps):
        res = h.resolve(0, t)
        h.check_bytes(res)
        err = h.attention(0, t, res)
        log(f"[tiny] step {t}: misses={int(res['stats']['n_miss'].sum())} attn max abs err {err[0]:.2e}")
    h.close()


def _small_store(R, ctx, B, T, Q, k, S, row_elems=576, page_rows=0, opt_pool_pages=0, sources=1):
    w_rows = row_elems * 2
    st = hsk.KVStore(requests=R, sources=sources, row_bytes=w_rows, hot_slots=B, tail_rows=T, ctx=ctx,
                     page_rows=page_rows, opt_pool_pages=opt_pool_pages, max_queries=Q, top_k=k, staging_rows=S)
    ora = [oracle.Source(R=R, ctx=ctx, B=B, T=T, page_rows=page_rows, opt_pool_pages=opt_pool_pages,
                         staging_rows=S, row_bytes=w_rows) for _ in range(sources)]
    w = synth.WORKLOADS["tiny"].scaled(row_elems=row_elems, seed=777)
    for s in range(sources):
        for r in range(R):
            synth.fill_kv_rows(st.host_ptr(s, r), w, s, r, 0, int(np.max(ctx)))
        ora[s].commit_prefill()
    st.commit_prefill()
    return st, ora, w


def _compare(st, ora, src, e, sel, nq=None):
    R = sel.shape[0]
    d_sel = torch.from_numpy(np.ascontiguousarray(sel)).cuda()
    d_nq = None if nq is None else torch.from_numpy(np.asarray(nq, np.int32)).cuda()
    d_locs = torch.full_like(d_sel, -7)
    d_stats = hsk.stats_tensor(R)
    st.resolve_step(src, e, d_sel, d_locs, d_stats, nq=d_nq)
    status = st.sync_status()
    locs = d_locs.cpu().numpy()
    stats = hsk.stats_to_numpy(d_stats)
    o = ora[src].resolve(e, sel, nq)
    assert np.array_equal(locs, o["locs"])
    for f in oracle.STATS_DTYPE.names:
        if f != "pad":
            assert np.array_equal(stats[f], o["stats"][f]), f
    for r in range(R):
        pos, dst = st.read_plan(src, r)
        assert np.array_equal(pos, o["plan"][r][0]) and np.array_equal(dst, o["plan"][r][1])
        g, a = st.snapshot(src, r), ora[src].snapshot(r)
        for key in ("key", "rec", "order", "pt", "opt"):
            assert np.array_equal(g[key], a[key]), (key, r)
    return d_locs, stats, status


def test_ragged_requests_partial_queries_duplicates_and_staging():
    """Ragged contexts, k not a multiple of any tile, per-request query counts (including 0), duplicate
    positions inside a query, tail rows, staging overflow within bounds, across 12 steps."""
    rng = np.random.default_rng(21)
    ctx = np.array([300, 1000, 64, 129, 4097], np.int64)
    R, B, T, Q, k, S = 5, 48, 16, 3, 37, 70
    st, ora, w = _small_store(R, ctx, B, T, Q, k, S)
    for t in range(12):
        sel = np.zeros((R, Q, k), np.int32)
        for r in range(R):
            sel[r] = rng.integers(0, ctx[r], size=(Q, k))
        nq = rng.integers(0, Q + 1, size=R).astype(np.int32)
        d_locs, stats, status = _compare(st, ora, 0, t + 1, sel, nq)
        assert status == 0
        # pool bytes at every emitted location equal the host row
        pool = st.pool_rows(0)
        for r in range(R):
            m = int(nq[r]) * k
            if m == 0:
                continue
            got = pool.index_select(0, d_locs[r].reshape(-1)[:m].long()).cpu().numpy()
            assert np.array_equal(got, st.host_rows(0, r)[sel[r].reshape(-1)[:m]])
    # attention with per-request query counts: skipped queries leave their outputs untouched
    H = 16
    q = rng.standard_normal((R, Q, H, 576)).astype(np.float32)
    q16 = torch.from_numpy(q).to(torch.bfloat16)
    out = torch.full((R, Q, H, 512), 77, dtype=torch.int16, device="cuda")
    ad = hsk.mla_desc(requests=R, max_queries=Q, heads=H, dk=576, dv=512, top_k=k, row_elems=576, scale=576 ** -0.5)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    d_nq = torch.from_numpy(nq).cuda()
    hsk.sparse_decode_attn(ad, q16.view(torch.int16).cuda(), st.pool_base(0), d_locs, d_nq, out, scratch, nb)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    qb = q16.view(torch.int16).numpy().view(np.uint16)
    for r in range(R):
        for j in range(Q):
            if j >= nq[r]:
                assert np.all(o[r, j] == 77)
                continue
            rows = synth.kv_rows_at(w, 0, r, sel[r, j])
            ref = oracle.mla_attention(qb[r, j], rows, 576, 512, 576 ** -0.5)
            g = synth.bf16_to_f32(o[r, j].view(np.uint16)).astype(np.float64)
            assert np.all(np.abs(g - ref) <= ATOL + RTOL * np.abs(ref))


def test_errors_are_reported_and_change_nothing():
    R, B, T, k = 3, 6, 2, 4
    ctx = np.array([50, 60, 70], np.int64)
    st, ora, w = _small_store(R, ctx, B, T, 2, k, 1)
    sel = np.array([[[1, 2, 3, 4], [1, 2, 3, 4]], [[1, 2, 3, 4], [1, 2, 3, 4]], [[9, 9, 9, 9], [10, 11, 12, 13]]],
                   np.int32)
    _compare(st, ora, 0, 1, sel)
    # request 0: a position equal to n_r (ERANGE); request 1: 8 new rows for 6 free slots + 1 staging row
    # (ESTAGE); request 2 unchanged
    bad = sel.copy()
    bad[0] = np.array([[1, 2, 3, 4], [5, 6, 7, 50]])
    bad[1] = np.array([[20, 21, 22, 23], [24, 25, 26, 27]])
    snaps = [st.snapshot(0, r) for r in range(R)]
    d_locs, stats, status = _compare(st, ora, 0, 2, bad)
    assert stats["status"][0] == hsk.HSK_ERANGE and stats["status"][1] == hsk.HSK_ESTAGE
    assert stats["status"][2] == 0
    assert status in (hsk.HSK_ERANGE, hsk.HSK_ESTAGE)
    loc = d_locs.cpu().numpy()
    assert np.all(loc[0] == -1) and np.all(loc[1] == -1)
    for r in (0, 1):
        for key in ("key", "rec", "order", "pt"):
            assert np.array_equal(st.snapshot(0, r)[key], snaps[r][key])
    assert st.sync_status() == 0  # cleared
    # negative position
    bad2 = sel.copy()
    bad2[2, 0, 0] = -3
    _, stats, status = _compare(st, ora, 0, 3, bad2)
    assert stats["status"][2] == hsk.HSK_ERANGE and status == hsk.HSK_ERANGE
    # epochs must increase: synchronous error, nothing queued
    d = torch.from_numpy(sel).cuda()
    with pytest.raises(hsk.HskError) as e:
        st.resolve_step(0, 3, d, torch.empty_like(d))
    assert e.value.status == hsk.HSK_EEPOCH
    st.close()


def test_direct_only_tail_selections_and_limits():
    """Every selection in the tail resolves directly and touches no hot metadata; a store at the maximum
    hot-cache size and the maximum selections per request stays exact."""
    R, B, T, k = 2, 16, 64, 32
    ctx = np.array([1000, 2000], np.int64)
    st, ora, w = _small_store(R, ctx, B, T, 1, k, 0)
    sel = np.stack([np.arange(ctx[r] - T, ctx[r] - T + k, dtype=np.int32)[None] for r in range(R)])
    d_locs, stats, _ = _compare(st, ora, 0, 1, sel)
    assert np.all(stats["n_tail"] == k) and np.all(stats["n_miss"] == 0)
    assert np.all(st.snapshot(0, 0)["key"] == -1)
    st.close()
    # limits
    R, B, Q, k = 2, hsk.MAX_HOT_SLOTS, 16, 4096
    ctx = np.array([200_000, 150_000], np.int64)
    st, ora, w = _small_store(R, ctx, B, 0, Q, k, Q * k, row_elems=64)
    rng = np.random.default_rng(3)
    for t in range(3):
        sel = np.stack([rng.integers(0, ctx[r], size=(Q, k)) for r in range(R)]).astype(np.int32)
        _, stats, status = _compare(st, ora, 0, t + 1, sel)
        assert status == 0
    st.close()


def test_optional_pages_and_reclaim_small():
    """Optional-history pages resolve directly; dropping them (reclaim) sends later selections through
    the hot cache and host gather; populating again publishes after the copy."""
    rng = np.random.default_rng(4)
    R, B, T, k, P = 4, 64, 8, 40, 16
    ctx = np.array([1000, 800, 1600, 640], np.int64)
    pages = ctx // P
    st, ora, w = _small_store(R, ctx, B, T, 1, k, 0, page_rows=P, opt_pool_pages=int(pages.sum()))
    nxt = 0
    ids = []
    for r in range(R):
        a = np.full(pages[r], -1, np.int32)
        keep = rng.choice(pages[r], size=pages[r] // 2, replace=False)
        a[keep] = nxt + np.arange(keep.size)
        nxt += keep.size
        ids.append(a)
        st.residency_set(0, r, a)
        assert ora[0].residency_set(r, a) == 0
    for t in range(10):
        if t == 5:
            for r in (0, 2):
                drop = np.full(pages[r], -1, np.int32)
                st.residency_set(0, r, drop)
                assert ora[0].residency_set(r, drop) == 0
        if t == 8:
            st.residency_set(0, 0, ids[0])
            assert ora[0].residency_set(0, ids[0]) == 0
        sel = np.stack([rng.choice(ctx[r], size=k, replace=False)[None] for r in range(R)]).astype(np.int32)
        d_locs, stats, status = _compare(st, ora, 0, t + 1, sel)
        pool = st.pool_rows(0)
        for r in range(R):
            got = pool.index_select(0, d_locs[r].reshape(-1).long()).cpu().numpy()
            assert np.array_equal(got, st.host_rows(0, r)[sel[r].reshape(-1)])
    st.close()


def test_dsa100k_full_size_sampled_attention():
    """The 100K-context batch-64 decode at full size (4 layers), in the launch configurations the
    benchmark times: resolve + gather + attention and the fused resolve + attend, alternating over
    (step, layer) on the same stores.  Resolution bit-exact on every call, pool bytes checked on every
    call, attention on sampled (request, layer, step) triples."""
    w = synth.WORKLOADS["dsa100k"]
    h = Harness(w, steps=4, check_meta_every=2)
    rng = np.random.default_rng(5)
    for t in range(h.steps):
        for layer in range(w.layers):
            fused = (t + layer) % 2 == 1
            res = h.resolve(layer, t, meta_reqs=range(0, w.requests, 9) if t % 2 == 0 else [], fused=fused)
            h.check_bytes(res)
            samples = [(int(r), 0) for r in rng.choice(w.requests, size=2, replace=False)]
            if fused:
                err = h.check_attention(layer, t, res, res["out"], samples=samples)
            else:
                err = h.attention(layer, t, res, samples=samples)
            st = res["stats"]
            log(f"[dsa100k] step {t} layer {layer} {'fused' if fused else 'separate'}: "
                f"hit_sel={int(st['n_hit_sel'].sum())} miss={int(st['n_miss'].sum())} "
                f"tail={int(st['n_tail'].sum())} attn err {err[0]:.2e}")
    h.close()


def test_verify_multiquery_union_and_staging():
    """Speculative verification: 16 queries per request share 60% of their rows; each distinct missing
    row is fetched once and unions beyond the free slots go to staging."""
    w = synth.WORKLOADS["verify"].scaled(requests=12)
    h = Harness(w, steps=4)
    for t in range(h.steps):
        res = h.resolve(0, t)
        h.check_bytes(res)
        st = res["stats"]
        assert np.all(st["n_miss"] <= st["n_miss_sel"])
        samples = [(r, j) for r in (0, 5, 11) for j in (0, 7, 15)]
        err = h.attention(0, t, res, samples=samples)
        log(f"[verify] step {t}: miss_sel={int(st['n_miss_sel'].sum())} distinct={int(st['n_miss'].sum())} "
            f"staged={int(st['n_staged'].sum())} attn err {err[0]:.2e}")
    h.close()


def test_adaptive_residency_and_reclaim():
    """Load-adaptive residency on a shared source read by two layers, with a reclaim of whole requests
    (Eq. 4) mid-run; the host-fetch fraction is reported before and after."""
    w = synth.WORKLOADS["adaptive"].scaled(requests=12, reclaim_requests=4, steps=8, reclaim_step=4)
    h = Harness(w, steps=w.steps)
    fetch = []
    for t in range(h.steps):
        if t == w.reclaim_step:
            h.reclaim()
        tot_miss = tot_sel = 0
        for layer in range(w.layers):
            res = h.resolve(layer, t, meta_reqs=range(0, w.requests, 3))
            h.check_bytes(res)
            if t in (0, w.reclaim_step):
                h.attention(layer, t, res, samples=[(0, 0), (7, 0)])
            tot_miss += int(res["stats"]["n_miss"].sum())
            tot_sel += int(res["stats"]["n_sel"].sum())
            assert int(res["stats"]["n_opt"].sum()) >= 0
        fetch.append(tot_miss / tot_sel)
        log(f"[adaptive] step {t}: host-fetch fraction {fetch[-1]:.4f}")
    h.close()


def test_quest_pages_plan_replay_side_stream():
    """Page-level GQA: layer 0 resolves, layers 1..7 replay its miss plan on a side stream ordered by
    events, and each layer's attention reads its own pool at layer 0's locations."""
    w = synth.WORKLOADS["quest"].scaled(requests=4)
    h = Harness(w, steps=3)
    side = torch.cuda.Stream()
    for t in range(h.steps):
        res = h.resolve(0, t)
        h.check_bytes(res, source=0)
        ev = torch.cuda.Event()
        ev.record()
        done = []
        with torch.cuda.stream(side):
            side.wait_event(ev)
            for layer in range(1, w.layers):
                h.store.replay_plan(0, layer, stream=side)
                e = torch.cuda.Event()
                e.record(side)
                done.append(e)
        for layer in range(w.layers):
            if layer:
                torch.cuda.current_stream().wait_event(done[layer - 1])
            err = h.attention(layer, t, res, samples=[0, 5, 17, 31], source=layer)
            if layer in (0, w.layers - 1):
                h.check_bytes(res, source=layer)
        log(f"[quest] step {t}: misses={int(res['stats']['n_miss'].sum())} attn err {err[0]:.2e}")
    h.close()
