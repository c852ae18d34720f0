"""GPU parity of the fused resolve + attend call (hsk_resolve_attend) through the C ABI.

Two identical stores run the same selections, one through hsk_resolve_step + hsk_sparse_decode_attn and
one through hsk_resolve_attend: locations, statistics, miss plans, metadata and pool bytes must be
identical; both attention outputs are checked against the CPU oracle (indexing bit-exact, attention
within 1e-2 + 2e-2 |ref|).  The outputs agree bit for bit where both calls run the same kernel (heads not
in multiples of 64); with heads in 64s the separate call runs the 32-heads-per-wave kernel, whose sums are
accumulated in another order.
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


def _pair(w, steps):
    return Harness(w, steps=steps), Harness(w, steps=steps)


# tiny: 16 heads (one 16-head block), k = 256; wide: 128 heads, k = 2048 with small batches (32-row
# partitions, many tiles of misses); ragged: k not a multiple of the 32-row tile; 256 heads: two head
# groups (only the first writes the fetched rows back); 48 heads: odd 16-head blocks
FUSED_CASES = {
    "tiny": dict(),
    "h128_k2048": dict(requests=2, ctx=30_000, hot_slots=4096, top_k=2048, heads=128, keep_frac=0.6),
    "h64_k300": dict(requests=3, ctx=5000, hot_slots=600, top_k=300, heads=64),
    "h256_k100": dict(requests=2, ctx=3000, hot_slots=256, top_k=100, heads=256),
    "h48_k129": dict(requests=5, ctx=4000, hot_slots=300, top_k=129, heads=48, fresh="zipf"),
}


@pytest.mark.parametrize("case", list(FUSED_CASES))
def test_fused_matches_unfused(case):
    w = synth.WORKLOADS["tiny"].scaled(**FUSED_CASES[case], seed=6100 + len(case))
    hu, hf = _pair(w, steps=5)
    for t in range(hu.steps):
        ru = hu.resolve(0, t)
        out_u = hu.run_attention(0, t, ru)
        rf = hf.resolve(0, t, fused=True)
        torch.cuda.synchronize()
        assert np.array_equal(ru["locs"], rf["locs"])
        for f in oracle.STATS_DTYPE.names:
            if f != "pad":
                assert np.array_equal(ru["stats"][f], rf["stats"][f]), f
        hf.check_bytes(rf)
        if w.heads % 64:
            assert torch.equal(out_u, rf["out"]), "fused output differs from resolve + attention"
        hu.check_attention(0, t, ru, out_u)
        err = hf.check_attention(0, t, rf, rf["out"])
        log(f"[fused {case}] step {t}: misses={int(rf['stats']['n_miss'].sum())} attn err {err[0]:.2e}")
    hu.close()
    hf.close()


def test_fused_duplicates_tail_and_rejected_request():
    """Duplicate positions inside a query (the first occurrence writes the row, the others read it from
    host), tail rows, and a request rejected for an out-of-range position next to good ones."""
    rng = np.random.default_rng(33)
    R, B, T, k, H = 4, 96, 16, 70, 32
    ctx = np.array([500, 2000, 129, 3000], np.int64)
    w_rows = 1152
    st = hsk.KVStore(requests=R, sources=1, row_bytes=w_rows, hot_slots=B, tail_rows=T, ctx=ctx, max_queries=1,
                     top_k=k)
    ora = oracle.Source(R=R, ctx=ctx, B=B, T=T, page_rows=0, opt_pool_pages=0, staging_rows=0, row_bytes=w_rows)
    w = synth.WORKLOADS["tiny"].scaled(seed=909)
    for r in range(R):
        synth.fill_kv_rows(st.host_ptr(0, r), w, 0, r, 0, int(ctx[r]))
    st.commit_prefill()
    ora.commit_prefill()
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=H, dk=576, dv=512, top_k=k, row_elems=576,
                      scale=576 ** -0.5)
    scratch = torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda")
    for t in range(6):
        sel = np.zeros((R, 1, k), np.int32)
        for r in range(R):
            base = rng.integers(0, ctx[r], size=k)
            base[k // 2:k // 2 + 6] = base[:6]           # duplicates of earlier entries
            base[-3:] = ctx[r] - 1 - np.arange(3)        # tail rows
            sel[r, 0] = base
        if t == 3:
            sel[2, 0, 5] = ctx[2]                        # out of range: request 2 is rejected
        q = rng.standard_normal((R, 1, H, 576)).astype(np.float32)
        q16 = torch.from_numpy(q).to(torch.bfloat16)
        d_sel = torch.from_numpy(sel).cuda()
        d_locs = torch.full_like(d_sel, -7)
        d_stats = hsk.stats_tensor(R)
        out = torch.zeros((R, 1, H, 512), dtype=torch.int16, device="cuda")
        st.resolve_attend(0, t + 1, d_sel, d_locs, ad, q16.view(torch.int16).cuda(), out, scratch, stats=d_stats)
        status = st.sync_status()
        o = ora.resolve(t + 1, sel)
        locs = d_locs.cpu().numpy()
        stats = hsk.stats_to_numpy(d_stats)
        assert np.array_equal(locs, o["locs"])
        for f in oracle.STATS_DTYPE.names:
            if f != "pad":
                assert np.array_equal(stats[f], o["stats"][f]), f
        if t == 3:
            assert stats["status"][2] == hsk.HSK_ERANGE and status == hsk.HSK_ERANGE
        pool = st.pool_rows(0)
        ob = out.cpu().numpy()
        qb = q16.view(torch.int16).numpy().view(np.uint16)
        for r in range(R):
            g, a = st.snapshot(0, r), ora.snapshot(r)
            for key in ("key", "rec", "order", "pt"):
                assert np.array_equal(g[key], a[key]), (key, r)
            if stats["status"][r] != 0:
                continue
            got = pool.index_select(0, d_locs[r].reshape(-1).long()).cpu().numpy()
            assert np.array_equal(got, st.host_rows(0, r)[sel[r].reshape(-1)])
            rows = synth.kv_rows_at(w, 0, r, sel[r, 0])
            ref = oracle.mla_attention(qb[r, 0], rows, 576, 512, 576 ** -0.5)
            gv = synth.bf16_to_f32(ob[r, 0].view(np.uint16)).astype(np.float64)
            assert np.all(np.abs(gv - ref) <= ATOL + RTOL * np.abs(ref)), f"r={r} t={t}"
    st.close()


def test_fused_rejects_shapes_and_changes_nothing():
    """Stores with several queries per request, no host reads, a descriptor that does not match the store
    or partitions above 1,024 rows are rejected before anything is queued: the epoch stays usable."""
    w = synth.WORKLOADS["tiny"].scaled(requests=2, top_k=2048, hot_slots=4096, ctx=20_000, heads=16, seed=5)
    h = Harness(w, steps=2)
    q, ad, out, scratch = h._attn_inputs(0, 0)
    sel = torch.from_numpy(h.sel[0][0]).cuda()
    locs = torch.empty_like(sel)
    bad = [hsk.mla_desc(requests=2, max_queries=1, heads=16, dk=576, dv=512, top_k=2048, row_elems=576,
                        scale=0.04, split=1),                      # 2,048-row partitions
           hsk.mla_desc(requests=3, max_queries=1, heads=16, dk=576, dv=512, top_k=2048, row_elems=576,
                        scale=0.04),                               # another batch
           hsk.mla_desc(requests=2, max_queries=1, heads=16, dk=576, dv=512, top_k=1024, row_elems=576,
                        scale=0.04)]                               # another k
    for d in bad:
        with pytest.raises(hsk.HskError) as e:
            h.store.resolve_attend(0, 1, sel, locs, d, q, out, scratch)
        assert e.value.status == hsk.HSK_EINVAL
    # the same epoch then works, and matches the oracle
    res = h.resolve(0, 0, fused=True)
    h.check_bytes(res)
    h.check_attention(0, 0, res, res["out"])
    h.close()
    st = hsk.KVStore(requests=2, sources=1, row_bytes=1152, hot_slots=64, tail_rows=4, ctx=1000, max_queries=2,
                     top_k=8)
    ad2 = hsk.mla_desc(requests=2, max_queries=1, heads=16, dk=576, dv=512, top_k=8, row_elems=576, scale=0.04)
    s2 = torch.empty(hsk.attn_scratch_bytes(ad2), dtype=torch.uint8, device="cuda")
    d = torch.zeros((2, 2, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(hsk.HskError) as e:
        st.resolve_attend(0, 1, d, torch.empty_like(d), ad2, torch.zeros((2, 16, 576), dtype=torch.int16,
                                                                          device="cuda"),
                          torch.zeros((2, 16, 512), dtype=torch.int16, device="cuda"), s2)
    assert e.value.status == hsk.HSK_EINVAL
    st.close()
    st = hsk.KVStore(requests=2, sources=1, row_bytes=1152, hot_slots=64, tail_rows=4, ctx=1000, max_queries=1,
                     top_k=8, gather_mode=hsk.GATHER_NO_IO)
    d = torch.zeros((2, 1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(hsk.HskError) as e:
        st.resolve_attend(0, 1, d, torch.empty_like(d), ad2, torch.zeros((2, 16, 576), dtype=torch.int16,
                                                                          device="cuda"),
                          torch.zeros((2, 16, 512), dtype=torch.int16, device="cuda"), s2)
    assert e.value.status == hsk.HSK_EINVAL
    st.close()
