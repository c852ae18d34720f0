"""GPU parity of the deferred fetch (HSK_GATHER_DEFERRED + hsk_fetch_plan) through the C ABI.

HiSparse section 3.5 splits a resolve into a plan and its IO; with a deferred store the resolve call plans
only and hsk_fetch_plan copies the plan's rows on a side stream, ordered by events.  Everything the
zero-copy resolve produces must come out the same: locations, statistics, plans and metadata bit-exact
against the oracle, pool bytes equal to the host rows at every emitted location (Adaptive DHiSparse
Eq. 12), attention within 1e-2 + 2e-2 |ref| of the fp64 oracle.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_sparse_kv_layer_amd as hsk  # noqa: E402
import synth  # noqa: E402
from hsk_harness import Harness, log  # noqa: E402


@pytest.mark.parametrize("gather_blocks", [1, 16, 18])
def test_deferred_fetch_matches_oracle(gather_blocks):
    """Single-query decode with duplicates of the tail and a ragged k: every call's misses fetched on a side
    stream by 1, 16 or 18 copy workgroups."""
    w = synth.WORKLOADS["tiny"].scaled(requests=5, top_k=129, hot_slots=300, heads=64, seed=7100 + gather_blocks)
    h = Harness(w, steps=6, gather_blocks=gather_blocks, deferred=True)
    for t in range(h.steps):
        res = h.resolve(0, t)
        h.check_bytes(res)
        err = h.attention(0, t, res)
        log(f"[fetch G={gather_blocks}] step {t}: misses={int(res['stats']['n_miss'].sum())} attn err {err[0]:.2e}")
    h.close()


def test_deferred_fetch_multiquery_staging():
    """Verification-shaped calls: 16 queries per request sharing 60% of their rows, unions beyond the hot
    slots staged; the fetch copies hot fills and staged rows alike."""
    w = synth.WORKLOADS["verify"].scaled(requests=6, ctx=40_000)
    h = Harness(w, steps=3, deferred=True)
    for t in range(h.steps):
        res = h.resolve(0, t)
        h.check_bytes(res)
        st = res["stats"]
        err = h.attention(0, t, res, samples=[(0, 0), (3, 9), (5, 15)])
        log(f"[fetch verify] step {t}: distinct={int(st['n_miss'].sum())} staged={int(st['n_staged'].sum())} "
            f"attn err {err[0]:.2e}")
    h.close()


def test_deferred_fetch_shared_staging_arena():
    """Three layers take turns in one shared staging arena (8 queries per request, unions overflowing into
    staging every step): each layer's fetch writes its staged rows into the arena at the rows its resolve
    emitted, checked against the oracle and the host rows before the next layer reuses the arena."""
    w = synth.WORKLOADS["verify"].scaled(requests=6, layers=3, sources=3, ctx=20_000, queries=8, top_k=512,
                                         hot_slots=1024, staging_rows=8 * 512, seed=7300)
    h = Harness(w, steps=3, staging_arenas=1, deferred=True)
    staged = 0
    for t in range(h.steps):
        for layer in range(w.layers):
            res = h.resolve(layer, t)
            h.check_bytes(res)
            staged += int(res["stats"]["n_staged"].sum())
            if t == h.steps - 1:
                h.attention(layer, t, res, samples=[(0, 0), (5, 7)])
    assert staged > 0, "the case must overflow into staging"
    log(f"[fetch arena] staged rows over the run: {staged}")
    h.close()


def test_deferred_fetch_full_size_layers():
    """The 100K-context batch-64 shape, 4 layers with their own payloads, 2 steps, with the copy kernel's
    18 workgroups (the launch the overlapped benchmark schedule uses)."""
    w = synth.WORKLOADS["dsa100k"]
    h = Harness(w, steps=2, gather_blocks=18, check_meta_every=2, deferred=True)
    rng = np.random.default_rng(17)
    for t in range(h.steps):
        for layer in range(w.layers):
            res = h.resolve(layer, t, meta_reqs=range(0, w.requests, 13))
            h.check_bytes(res)
            samples = [(int(r), 0) for r in rng.choice(w.requests, size=2, replace=False)]
            err = h.attention(layer, t, res, samples=samples)
            log(f"[fetch dsa100k] step {t} layer {layer}: miss={int(res['stats']['n_miss'].sum())} "
                f"attn err {err[0]:.2e}")
    h.close()


def test_fetch_errors():
    """hsk_fetch_plan needs a deferred store and a resolve on the source; a deferred store has no fused call;
    plan replay copies in deferred stores too."""
    kw = dict(requests=2, sources=2, row_bytes=1152, hot_slots=64, tail_rows=4, ctx=1000, max_queries=1, top_k=8)
    zc = hsk.KVStore(**kw)
    with pytest.raises(hsk.HskError) as e:
        zc.fetch_plan(0)
    assert e.value.status == hsk.HSK_EINVAL
    zc.close()
    st = hsk.KVStore(gather_mode=hsk.GATHER_DEFERRED, **kw)
    w = synth.WORKLOADS["tiny"].scaled(seed=31)
    for s in range(2):
        for r in range(2):
            synth.fill_kv_rows(st.host_ptr(s, r), w, s, r, 0, 1000)
    st.commit_prefill()
    with pytest.raises(hsk.HskError) as e:
        st.fetch_plan(0)                       # no resolve yet
    assert e.value.status == hsk.HSK_ESTATE
    for bad in (-1, 2):
        with pytest.raises(hsk.HskError) as e:
            st.fetch_plan(bad)
        assert e.value.status == hsk.HSK_EINVAL
    sel = torch.tensor([[[1, 2, 3, 4, 5, 6, 7, 8]], [[10, 20, 30, 40, 50, 60, 70, 80]]], dtype=torch.int32,
                       device="cuda")
    locs = torch.empty_like(sel)
    ad = hsk.mla_desc(requests=2, max_queries=1, heads=16, dk=576, dv=512, top_k=8, row_elems=576, scale=0.04)
    scratch = torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda")
    with pytest.raises(hsk.HskError) as e:
        st.resolve_attend(0, 1, sel, locs, ad, torch.zeros((2, 16, 576), dtype=torch.int16, device="cuda"),
                          torch.zeros((2, 16, 512), dtype=torch.int16, device="cuda"), scratch)
    assert e.value.status == hsk.HSK_EINVAL
    st.resolve_step(0, 1, sel, locs)
    st.fetch_plan(0)
    st.replay_plan(0, 1)                       # source 1 gets source 0's plan rows from its own host rows
    torch.cuda.synchronize()
    assert st.sync_status() == 0
    for s in range(2):
        pool = st.pool_rows(s)
        for r in range(2):
            got = pool.index_select(0, locs[r].reshape(-1).long()).cpu().numpy()
            assert np.array_equal(got, st.host_rows(s, r)[sel[r].reshape(-1).cpu().numpy()]), (s, r)
    st.close()


OVERLAP_CASES = {
    "tiny_mla16": ("tiny", dict(requests=5, top_k=129, hot_slots=300, heads=16)),
    "mla128_k2048": ("tiny", dict(requests=3, ctx=30_000, top_k=2048, hot_slots=4096, heads=128, keep_frac=0.6)),
    "verify_8q": ("verify", dict(requests=4, ctx=20_000, queries=8, top_k=512, hot_slots=1024, staging_rows=8 * 512)),
    "quest_gqa": ("quest", dict(requests=2, layers=1)),
}


@pytest.mark.parametrize("case", list(OVERLAP_CASES))
@pytest.mark.parametrize("same_stream", [False, True])
def test_resolve_fetch_attend(case, same_stream):
    """hsk_resolve_fetch_attend: resolve (plan only), fetch on the copy stream, attention after it, in one call:
    resolution bit-exact against the oracle, pool bytes equal to the host rows, attention within tolerance of the
    fp64 oracle; MLA with 16 and 128 heads, 8 queries per request with staging, GQA pages; copy stream distinct from
    or equal to the stream."""
    base, kw = OVERLAP_CASES[case]
    w = synth.WORKLOADS[base].scaled(**kw, seed=7400 + len(case))
    h = Harness(w, steps=3, deferred=True)
    for t in range(h.steps):
        res = h.resolve(0, t, overlap=True, same_stream=same_stream)
        h.check_bytes(res, source=0)
        if w.kind == "mla":
            samples = [(r, j) for r in range(min(w.requests, 3)) for j in (0, w.queries - 1)]
        else:
            samples = [0, 3, h.U - 1]
        err = h.check_attention(0, t, res, res["out"], samples=samples, source=0)
        log(f"[overlap {case}] step {t}: misses={int(res['stats']['n_miss'].sum())} attn err {err[0]:.2e}")
    h.close()


def test_resolve_fetch_attend_copy_waits_for_a_late_resolve():
    """With the copy on its own stream, the copy kernel is not ordered after the resolve by the streams: it waits
    inside for each request's published plan.  Here ~10 ms of matrix products run on the stream before every
    call, so the copy stream (idle) starts the copy kernel long before the resolve runs: the pool must still get
    exactly the plan's rows (at the first step a copy that did not wait would read the initial empty plan), and
    no copy may give up waiting (error word clear)."""
    w = synth.WORKLOADS["tiny"].scaled(requests=3, ctx=30_000, top_k=2048, hot_slots=4096, heads=128, keep_frac=0.6,
                                       seed=7450)
    h = Harness(w, steps=3, deferred=True)
    a = torch.randn(4096, 4096, device="cuda")
    for t in range(h.steps):
        torch.cuda.synchronize()
        for _ in range(6):
            a = a @ a
            a = a / a.norm()
        res = h.resolve(0, t, overlap=True)
        h.check_bytes(res, source=0)
        err = h.check_attention(0, t, res, res["out"], samples=[(r, 0) for r in range(w.requests)], source=0)
        log(f"[late resolve] step {t}: misses={int(res['stats']['n_miss'].sum())} attn err {err[0]:.2e}")
    assert h.store.sync_status() == 0
    h.close()


def test_resolve_fetch_attend_rejects_and_changes_nothing():
    """A zero-copy store, a descriptor for another batch, k or row width, and too little scratch are rejected
    before anything is queued: the same epoch then works."""
    w = synth.WORKLOADS["tiny"].scaled(requests=2, top_k=64, hot_slots=128, heads=16, seed=77)
    h = Harness(w, steps=2, deferred=True)
    q, ad, out, scratch = h._attn_inputs(0, 0)
    sel = torch.from_numpy(h.sel[0][0]).cuda()
    locs = torch.empty_like(sel)
    bad = [hsk.mla_desc(requests=3, max_queries=1, heads=16, dk=576, dv=512, top_k=64, row_elems=576, scale=0.04),
           hsk.mla_desc(requests=2, max_queries=1, heads=16, dk=576, dv=512, top_k=32, row_elems=576, scale=0.04),
           hsk.mla_desc(requests=2, max_queries=1, heads=16, dk=576, dv=512, top_k=64, row_elems=584, scale=0.04)]
    for d in bad:
        with pytest.raises(hsk.HskError) as e:
            h.store.resolve_fetch_attend(0, 1, sel, locs, d, q, out, scratch)
        assert e.value.status == hsk.HSK_EINVAL
    with pytest.raises(hsk.HskError) as e:
        h.store.resolve_fetch_attend(0, 1, sel, locs, ad, q, out, scratch[:128])
    assert e.value.status == hsk.HSK_EINVAL
    res = h.resolve(0, 0, overlap=True)
    h.check_bytes(res)
    h.check_attention(0, 0, res, res["out"])
    h.close()
    zc = hsk.KVStore(requests=2, sources=1, row_bytes=1152, hot_slots=128, tail_rows=64, ctx=8192, max_queries=1,
                     top_k=64)
    with pytest.raises(hsk.HskError) as e:
        zc.resolve_fetch_attend(0, 1, sel, locs, ad, q, out, scratch)
    assert e.value.status == hsk.HSK_EINVAL
    zc.close()


def test_resolve_fetch_attend_query_counts_match_separate_calls():
    """Per-request query counts (nq = 1, 3, 0, 2 of Qmax = 3): a deferred store through hsk_resolve_fetch_attend
    and a zero-copy store through hsk_resolve_step + hsk_sparse_decode_attn, same inputs, give identical
    locations and statistics, identical pool bytes at every location, and bit-identical attention outputs
    (same kernel, same partitions, same rows) for the queries that exist; the skipped queries' outputs stay
    untouched."""
    R, Q, k, B, T, n = 4, 3, 96, 512, 16, 3000   # B >= Q k: no union overflows, no request is rejected
    w = synth.WORKLOADS["tiny"].scaled(requests=R, queries=Q, top_k=k, hot_slots=B, tail_rows=T, ctx=n, heads=64,
                                       seed=7700)
    kw = dict(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=B, tail_rows=T, ctx=n, max_queries=Q, top_k=k)
    zc = hsk.KVStore(**kw)
    df = hsk.KVStore(gather_mode=hsk.GATHER_DEFERRED, **kw)
    for st in (zc, df):
        for r in range(R):
            synth.fill_kv_rows(st.host_ptr(0, r), w, 0, r, 0, n)
        st.commit_prefill()
    nq = torch.tensor([1, 3, 0, 2], dtype=torch.int32, device="cuda")
    ad = hsk.mla_desc(requests=R, max_queries=Q, heads=64, dk=576, dv=512, top_k=k, row_elems=576, scale=576 ** -0.5)
    nb = hsk.attn_scratch_bytes(ad)
    sc = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    copy = torch.cuda.Stream()
    sels = synth.selection_stream(w, 0, steps=4)
    for t in range(4):
        sel = torch.from_numpy(sels[t]).cuda()
        q = torch.from_numpy(synth.queries(w, 0, t).view(np.int16)).cuda()
        outs = [torch.full((R, Q, 64, 512), 77, dtype=torch.int16, device="cuda") for _ in range(2)]
        locs = [torch.full_like(sel, -7) for _ in range(2)]
        stats = [hsk.stats_tensor(R) for _ in range(2)]
        zc.resolve_step(0, t + 1, sel, locs[0], stats[0], nq=nq)
        hsk.sparse_decode_attn(ad, q, zc.pool_base(0), locs[0], nq, outs[0], sc[0], nb)
        df.resolve_fetch_attend(0, t + 1, sel, locs[1], ad, q, outs[1], sc[1], stats=stats[1], nq=nq,
                                copy_stream=copy)
        torch.cuda.synchronize()
        assert zc.sync_status() == 0 and df.sync_status() == 0
        assert torch.equal(locs[0], locs[1])
        s0, s1 = hsk.stats_to_numpy(stats[0]), hsk.stats_to_numpy(stats[1])
        for f in s0.dtype.names:
            if f != "pad":
                assert np.array_equal(s0[f], s1[f]), f
        for r in range(R):
            m = int(nq[r])
            if m == 0:
                continue
            rows = locs[1][r, :m].reshape(-1).long()
            assert torch.equal(zc.pool_rows(0).index_select(0, rows), df.pool_rows(0).index_select(0, rows))
            assert torch.equal(outs[0][r, :m], outs[1][r, :m]), (t, r)
            assert bool((outs[1][r, m:] == 77).all()), "a skipped query's output was written"
    zc.close()
    df.close()


def test_resolve_fetch_attend_rejected_request_reads_inside_the_pool():
    """A request whose union overflows the hot slots with no staging rows is rejected (ESTAGE, locations -1);
    the call's attention still runs over the batch: the rejected request's locations are read as row 0 (no
    load outside the pool), and every other request's output equals the separate calls' on a zero-copy store."""
    R, Q, k, B, T, n = 3, 3, 96, 256, 16, 3000
    w = synth.WORKLOADS["tiny"].scaled(requests=R, queries=Q, top_k=k, hot_slots=B, tail_rows=T, ctx=n, heads=64,
                                       seed=7700)
    sel_np = synth.selection_stream(w, 0, steps=1)[0].copy()
    # request 1: three disjoint lists of 96 rows below the tail -> a 288-row union against 256 slots; requests
    # 0 and 2 use one query each (95 distinct rows)
    sel_np[1] = np.arange(3 * k, dtype=np.int32).reshape(Q, k) + 100
    nq = torch.tensor([1, 3, 1], dtype=torch.int32, device="cuda")
    kw = dict(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=B, tail_rows=T, ctx=n, max_queries=Q, top_k=k)
    zc = hsk.KVStore(**kw)
    df = hsk.KVStore(gather_mode=hsk.GATHER_DEFERRED, **kw)
    for st in (zc, df):
        for r in range(R):
            synth.fill_kv_rows(st.host_ptr(0, r), w, 0, r, 0, n)
        st.commit_prefill()
    ad = hsk.mla_desc(requests=R, max_queries=Q, heads=64, dk=576, dv=512, top_k=k, row_elems=576, scale=576 ** -0.5)
    nb = hsk.attn_scratch_bytes(ad)
    sc = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sel = torch.from_numpy(sel_np).cuda()
    q = torch.from_numpy(synth.queries(w, 0, 0).view(np.int16)).cuda()
    outs = [torch.zeros((R, Q, 64, 512), dtype=torch.int16, device="cuda") for _ in range(2)]
    locs = [torch.full_like(sel, -7) for _ in range(2)]
    stats = [hsk.stats_tensor(R) for _ in range(2)]
    zc.resolve_step(0, 1, sel, locs[0], stats[0], nq=nq)
    hsk.sparse_decode_attn(ad, q, zc.pool_base(0), locs[0], nq, outs[0], sc[0], nb)
    df.resolve_fetch_attend(0, 1, sel, locs[1], ad, q, outs[1], sc[1], stats=stats[1], nq=nq,
                            copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert zc.sync_status() == hsk.HSK_ESTAGE and df.sync_status() == hsk.HSK_ESTAGE
    s1 = hsk.stats_to_numpy(stats[1])
    assert s1["status"][1] == hsk.HSK_ESTAGE and s1["status"][0] == 0 and s1["status"][2] == 0
    assert torch.equal(locs[0], locs[1]) and bool((locs[1][1] == -1).all())
    for r in (0, 2):
        assert torch.equal(outs[0][r, 0], outs[1][r, 0]), r
    zc.close()
    df.close()


def test_fetch_edge_cases():
    """One request; a call whose rows are all hits (an empty plan: the fetch copies nothing and the pool keeps its
    bytes); the same plan fetched twice (the second copy writes the same bytes again)."""
    w = synth.WORKLOADS["tiny"].scaled(requests=1, top_k=64, hot_slots=128, heads=16, seed=7800)
    h = Harness(w, steps=1, deferred=True)
    res = h.resolve(0, 0)                          # cold: every non-tail row misses
    h.check_bytes(res)
    assert int(res["stats"]["n_miss"].sum()) > 0
    sel = torch.from_numpy(h.sel[0][0]).cuda()
    locs = torch.empty_like(sel)
    stats = hsk.stats_tensor(1)
    before = h.store.pool_rows(0).clone()
    h.store.resolve_step(0, 2, sel, locs, stats)   # the same selection again: all hits
    h.store.fetch_plan(0)
    torch.cuda.synchronize()
    assert h.store.sync_status() == 0
    st = hsk.stats_to_numpy(stats)
    assert int(st["n_miss"][0]) == 0 and int(st["n_hit_sel"][0]) + int(st["n_tail"][0]) == w.top_k
    assert torch.equal(before, h.store.pool_rows(0)), "an empty plan changed the pool"
    assert h.store.read_plan(0, 0)[0].size == 0
    # a new selection with misses, fetched twice
    sel2 = torch.from_numpy(((h.sel[0][0] + 997) % (w.ctx - w.tail_rows)).astype(np.int32)).cuda()
    h.store.resolve_step(0, 3, sel2, locs, stats)
    h.store.fetch_plan(0)
    h.store.fetch_plan(0)
    torch.cuda.synchronize()
    assert h.store.sync_status() == 0 and int(hsk.stats_to_numpy(stats)["n_miss"][0]) > 0
    got = h.store.pool_rows(0).index_select(0, locs.reshape(-1).long()).cpu().numpy()
    assert np.array_equal(got, h.store.host_rows(0, 0)[sel2.cpu().numpy().reshape(-1)])
    h.close()


def test_overlapped_calls_on_dedicated_streams():
    """hsk_stream_create streams (hardware queues of their own) for the micro-batch streams and the copy stream:
    two stores' calls interleaved as in the overlapped schedule, each checked against its oracle."""
    ws = [synth.WORKLOADS["tiny"].scaled(requests=3, top_k=256, hot_slots=512, heads=64, seed=7900 + i)
          for i in range(2)]
    hs = [Harness(w, steps=3, deferred=True) for w in ws]
    *streams, copy = hsk.dedicated_streams(len(hs) + 1)
    for h in hs:
        h.copy_stream = copy
    for t in range(3):
        for h, s in zip(hs, streams):
            with torch.cuda.stream(s):
                res = h.resolve(0, t, overlap=True)
                h.check_bytes(res)
                h.check_attention(0, t, res, res["out"])
    for h in hs:
        h.close()
