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


@pytest.mark.parametrize("gather_blocks", [1, 16])
def test_deferred_fetch_matches_oracle(gather_blocks):
    """Single-query decode with duplicates of the tail and a ragged k: every call's misses fetched on a side
    stream by 1 or 16 copy workgroups."""
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
    16 workgroups (the launch the overlapped benchmark schedule uses)."""
    w = synth.WORKLOADS["dsa100k"]
    h = Harness(w, steps=2, gather_blocks=16, check_meta_every=2, deferred=True)
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
