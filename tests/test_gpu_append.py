"""GPU parity of the decode-loop append (hsk_append_rows) through the C ABI against the CPU oracle.

Every step appends new rows to each source (tail ring on the main stream, write-through to the pinned host
rows on a second stream), then resolves selections that include the newest rows and rows that have just left
the tail.  Locations, statistics, miss plans and metadata must equal the oracle's; the pool bytes at every
location must be the selected row; the host rows of the appended positions must hold the appended rows after
the write-through (they start as a sentinel); attention over the result matches the fp64 oracle.
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
from hsk_harness import log, ATOL, RTOL  # noqa: E402

SENTINEL = 0x5A


def _store(R, ctx, max_ctx, B, T, k, sources, seed):
    w = synth.WORKLOADS["tiny"].scaled(seed=seed)
    st = hsk.KVStore(requests=R, sources=sources, row_bytes=w.row_bytes, hot_slots=B, tail_rows=T, ctx=ctx,
                     max_ctx=max_ctx, max_queries=1, top_k=k)
    for s in range(sources):
        for r in range(R):
            h = st.host_rows(s, r)
            h[:] = SENTINEL
            synth.fill_kv_rows(st.host_ptr(s, r), w, s, r, 0, int(ctx[r]))
    st.commit_prefill()
    ora = [oracle.Source(R=R, ctx=ctx, B=B, T=T, row_bytes=w.row_bytes, max_ctx=max_ctx) for _ in range(sources)]
    for o in ora:
        o.commit_prefill()
    torch.cuda.synchronize()
    return st, ora, w


def _check_resolve(st, o_src, src, epoch, sel, w, n):
    d_sel = torch.from_numpy(sel).cuda()
    d_locs = torch.full_like(d_sel, -7)
    d_stats = hsk.stats_tensor(sel.shape[0])
    st.resolve_step(src, epoch, d_sel, d_locs, d_stats)
    assert st.sync_status() == 0
    locs = d_locs.cpu().numpy()
    stats = hsk.stats_to_numpy(d_stats)
    o = o_src.resolve(epoch, sel)
    assert o["rc"] == 0
    assert np.array_equal(locs, o["locs"]), "locations differ"
    for f in oracle.STATS_DTYPE.names:
        if f != "pad":
            assert np.array_equal(stats[f], o["stats"][f]), f
    pool = st.pool_rows(src)
    for r in range(sel.shape[0]):
        pos, dst = st.read_plan(src, r)
        assert np.array_equal(pos, o["plan"][r][0]) and np.array_equal(dst, o["plan"][r][1])
        g, a = st.snapshot(src, r), o_src.snapshot(r)
        for key in ("key", "rec", "order", "pt"):
            assert np.array_equal(g[key], a[key]), (key, r)
        got = pool.index_select(0, d_locs[r].reshape(-1).long()).cpu().numpy()
        want = synth.kv_rows_at(w, src, r, sel[r].reshape(-1)).view(np.uint8).reshape(got.shape)
        assert np.array_equal(got, want), f"pool bytes differ from the selected rows, request {r}"
    return d_locs, stats


@pytest.mark.parametrize("same_stream", [False, True])
def test_append_tail_write_through_and_history(same_stream):
    rng = np.random.default_rng(17)
    R, B, T, k, S = 5, 48, 8, 37, 2
    ctx = np.array([300, 1000, 64, 129, 4097], np.int64)
    max_ctx = int(ctx.max()) + 200
    st, ora, w = _store(R, ctx, max_ctx, B, T, k, S, seed=71)
    main = torch.cuda.current_stream()
    backup = main if same_stream else torch.cuda.Stream()
    n = [ctx.copy() for _ in range(S)]
    for t in range(14):
        c = 1 + t % (T // 2)
        for s in range(S):
            # the layer's new rows for positions n_r .. n_r + c - 1 (deterministic per position)
            rows = np.stack([synth.kv_rows(w, s, r, int(n[s][r]), c) for r in range(R)])
            d_rows = torch.from_numpy(rows.view(np.int16)).cuda()
            st.append_rows(s, d_rows, c, stream=main, backup_stream=backup)
            assert ora[s].append(c) == 0
            n[s] += c
            for r in range(R):
                assert st.context_rows(s, r) == int(n[s][r]) == ora[s].context_rows(r)
            # newest rows, rows that just left the tail, and random history
            sel = np.zeros((R, 1, k), np.int32)
            for r in range(R):
                nr = int(n[s][r])
                newest = np.arange(nr - c, nr)
                left = np.arange(max(0, nr - T - c), nr - T)
                rest = rng.choice(nr, size=k, replace=False)
                pick = np.concatenate([newest, left, rest[~np.isin(rest, np.concatenate([newest, left]))]])[:k]
                sel[r, 0] = pick
            _check_resolve(st, ora[s], s, t + 1, sel, w, n[s])
    torch.cuda.synchronize()
    # write-through: every appended position's host row holds the appended row
    for s in range(S):
        for r in range(R):
            lo, hi = int(ctx[r]), int(n[s][r])
            got = st.host_rows(s, r)[lo:hi]
            want = synth.kv_rows(w, s, r, lo, hi - lo).view(np.uint8).reshape(got.shape)
            assert np.array_equal(got, want), f"host rows of source {s} request {r} not written through"
            assert np.all(st.host_rows(s, r)[hi:hi + 1] == SENTINEL)
    log(f"[append] same_stream={same_stream}: 14 steps x {S} sources exact")
    st.close()


def test_append_decode_loop_attention():
    """A short decode loop: append one row per request, resolve the newest rows with Zipf history, attend;
    attention over the result equals the fp64 oracle over the selected rows (the appended ones included)."""
    R, B, T, k, H = 4, 64, 4, 48, 32
    ctx = np.array([500, 2000, 129, 3000], np.int64)
    st, ora, w = _store(R, ctx, int(ctx.max()) + 64, B, T, k, 1, seed=72)
    rng = np.random.default_rng(9)
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=H, dk=576, dv=512, top_k=k, row_elems=576, scale=576 ** -0.5)
    scratch = torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda")
    n = ctx.copy()
    backup = torch.cuda.Stream()
    for t in range(10):
        rows = np.stack([synth.kv_rows(w, 0, r, int(n[r]), 1) for r in range(R)])
        st.append_rows(0, torch.from_numpy(rows.view(np.int16)).cuda(), 1, backup_stream=backup)
        assert ora[0].append(1) == 0
        n += 1
        sel = np.stack([np.concatenate([[n[r] - 1], rng.choice(int(n[r]) - 1, size=k - 1, replace=False)])
                        for r in range(R)]).astype(np.int32)[:, None]
        d_locs, _ = _check_resolve(st, ora[0], 0, t + 1, sel, w, n)
        q = torch.from_numpy(rng.standard_normal((R, 1, H, 576)).astype(np.float32)).to(torch.bfloat16)
        out = torch.zeros((R, 1, H, 512), dtype=torch.int16, device="cuda")
        hsk.sparse_decode_attn(ad, q.view(torch.int16).cuda(), st.pool_base(0), d_locs, None, out, scratch,
                               scratch.numel())
        ob = out.cpu().numpy()
        qb = q.view(torch.int16).numpy().view(np.uint16)
        for r in range(R):
            ref = oracle.mla_attention(qb[r, 0], synth.kv_rows_at(w, 0, r, sel[r, 0]), 576, 512, 576 ** -0.5)
            g = synth.bf16_to_f32(ob[r, 0].view(np.uint16)).astype(np.float64)
            assert np.all(np.abs(g - ref) <= ATOL + RTOL * np.abs(ref)), f"t={t} r={r}"
    st.close()


def test_append_rejections_change_nothing():
    R, B, T, k = 2, 8, 4, 4
    ctx = np.array([10, 17], np.int64)
    st, ora, w = _store(R, ctx, 20, B, T, k, 1, seed=73)
    rows = torch.zeros((R, 3, w.row_elems), dtype=torch.int16, device="cuda")
    for count in (0, 3):                          # 2 count > T
        with pytest.raises(hsk.HskError) as e:
            st.append_rows(0, rows, count)
        assert e.value.status == hsk.HSK_EINVAL
    st.append_rows(0, rows, 2)                    # 12, 19
    with pytest.raises(hsk.HskError) as e:        # request 1 would pass max_ctx
        st.append_rows(0, rows, 2)
    assert e.value.status == hsk.HSK_EINVAL
    assert [st.context_rows(0, r) for r in range(R)] == [12, 19]
    st.close()
    al = hsk.KVStore(requests=1, sources=2, row_bytes=1152, hot_slots=4, tail_rows=4, ctx=8, max_ctx=16, top_k=2,
                     host_alias=True)
    with pytest.raises(hsk.HskError) as e:
        al.append_rows(0, torch.zeros((1, 1, 576), dtype=torch.int16, device="cuda"), 1)
    assert e.value.status == hsk.HSK_EINVAL
    al.close()
