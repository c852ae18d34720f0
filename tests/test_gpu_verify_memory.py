"""GPU parity of the verification memory path through the C ABI: staging arenas shared by the sources
(Adaptive DHiSparse section 3.4, reused by the next layer group once its readers are done)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_sparse_kv_layer_amd as hsk  # noqa: E402
import synth  # noqa: E402
from hsk_harness import Harness, log  # noqa: E402


@pytest.mark.parametrize("arenas", [1, 2])
def test_shared_staging_arenas(arenas):
    """Three layers with their own payloads take turns in `arenas` staging arenas: 8 queries per request
    share half their rows, unions overflow the hot cache into staging every step.  Every call is compared
    with the oracle bit for bit (staged locations included), pool bytes at every location are the selected
    rows, attention matches the fp64 oracle, and the pool is smaller than with one arena per source."""
    w = synth.WORKLOADS["verify"].scaled(requests=8, layers=3, sources=3, ctx=20_000, queries=8, top_k=512,
                                         hot_slots=1024, staging_rows=8 * 512, seed=3100 + arenas)
    h = Harness(w, steps=4, staging_arenas=arenas)
    st = h.store
    region = st.rows_per_source
    full = hsk.workspace_bytes(hsk.Desc(num_requests=8, num_sources=3, row_bytes=w.row_bytes, hot_slots=1024,
                                        tail_rows=w.tail_rows, max_queries=8, top_k=512, staging_rows=8 * 512,
                                        max_ctx=w.ctx, ctx_len=h.store.ctx.ctypes.data))[1]
    assert st.pool.numel() == full - (3 - arenas) * 8 * 8 * 512 * w.row_bytes
    staged_total = 0
    for t in range(h.steps):
        for layer in range(w.layers):
            res = h.resolve(layer, t)
            h.check_bytes(res)
            stats = res["stats"]
            staged_total += int(stats["n_staged"].sum())
            # staged locations lie in the layer's arena, after the last source region
            locs = res["locs"].reshape(-1)
            arena0 = w.sources * region + (layer % arenas) * 8 * 8 * 512 - layer * region
            outside = locs[locs >= region]
            assert np.all((outside >= arena0) & (outside < arena0 + 8 * 8 * 512))
            assert (outside.size > 0) == (int(stats["n_staged"].sum()) > 0)
            err = h.attention(layer, t, res, samples=[(0, 0), (3, 5), (7, 7)])
            log(f"[arenas={arenas}] step {t} layer {layer}: staged={int(stats['n_staged'].sum())} err {err[0]:.2e}")
    assert staged_total > 0
    h.close()


def test_replay_rejected_with_shared_staging():
    st = hsk.KVStore(requests=2, sources=2, row_bytes=1152, hot_slots=8, tail_rows=4, ctx=64, max_queries=2,
                     top_k=8, staging_rows=8, staging_arenas=1)
    with pytest.raises(hsk.HskError) as e:
        st.replay_plan(0, 1)
    assert e.value.status == hsk.HSK_EINVAL
    st.close()


def test_replay_destination_is_replay_only():
    """A replay destination's pool rows follow the plan source's slot table, so the library refuses to
    resolve it afterwards, to replay into a source that has resolved, to use a destination as a plan
    source, and to replay a source into itself."""
    st = hsk.KVStore(requests=2, sources=3, row_bytes=1152, hot_slots=8, tail_rows=4, ctx=64, max_queries=1,
                     top_k=8)
    sel = torch.zeros((2, 1, 8), dtype=torch.int32, device="cuda")
    sel[:, 0, :] = torch.arange(8, dtype=torch.int32)
    locs = torch.empty_like(sel)
    st.resolve_step(0, 1, sel, locs)
    with pytest.raises(hsk.HskError) as e:
        st.replay_plan(0, 0)
    assert e.value.status == hsk.HSK_EINVAL
    st.resolve_step(2, 1, sel, locs)
    with pytest.raises(hsk.HskError) as e:          # source 2 has its own metadata
        st.replay_plan(0, 2)
    assert e.value.status == hsk.HSK_ESTATE
    st.replay_plan(0, 1)
    with pytest.raises(hsk.HskError) as e:
        st.resolve_step(1, 2, sel, locs)
    assert e.value.status == hsk.HSK_ESTATE
    with pytest.raises(hsk.HskError) as e:
        st.replay_plan(1, 2)
    assert e.value.status == hsk.HSK_ESTATE
    st.replay_plan(0, 1)                             # replaying again into the same destination is fine
    assert st.sync_status() == 0
    st.close()


def test_draft_ring_write_window_and_attention():
    """Draft rows written round by round (blocks of up to K_max rows) wrap around a ring of R_d rows (Eq. 9);
    the window locations are Eq. 10's addresses, the ring rows at them hold the window's rows, and attention
    over the window matches the fp64 oracle."""
    import oracle
    rng = np.random.default_rng(31)
    slots, window, page, k_max, H = 3, 200, 16, 8, 16
    ring = hsk.ring_rows(window, page, k_max)
    assert ring == oracle.ring_rows(window, page, k_max)
    w = synth.WORKLOADS["tiny"].scaled(seed=3200)
    d_ring = torch.empty(slots * ring * w.row_bytes, dtype=torch.uint8, device="cuda")
    t = np.array([0, 5, 37], np.int64)          # each slot's next draft position
    ad = hsk.mla_desc(requests=slots, max_queries=1, heads=H, dk=576, dv=512, top_k=window, row_elems=576,
                      scale=576 ** -0.5)
    scratch = torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda")
    locs = torch.empty((slots, 1, window), dtype=torch.int32, device="cuda")
    checked = 0
    for rnd in range(70):
        count = int(rng.integers(1, k_max + 1))
        rows = np.stack([synth.kv_rows(w, 9, i, int(t[i]), count) for i in range(slots)])
        hsk.ring_write(d_ring, ring, slots, torch.from_numpy(rows.view(np.int16)).cuda(), count, w.row_bytes,
                       torch.from_numpy(t.copy()).cuda())
        t += count
        hsk.ring_window_locs(ring, slots, window, torch.from_numpy(t.copy()).cuda(), locs)
        lo = locs.cpu().numpy().reshape(slots, window)
        for i in range(slots):
            pos = np.arange(t[i] - window, t[i])
            want = np.array([oracle.ring_addr(i, int(p), ring) if p >= 0 else -1 for p in pos])
            assert np.array_equal(lo[i], want), f"round {rnd} slot {i}"
        if np.all(t >= window) and rnd % 10 == 9:
            view = d_ring.view(slots * ring, w.row_bytes)
            q = torch.from_numpy(rng.standard_normal((slots, 1, H, 576)).astype(np.float32)).to(torch.bfloat16)
            out = torch.zeros((slots, 1, H, 512), dtype=torch.int16, device="cuda")
            hsk.sparse_decode_attn(ad, q.view(torch.int16).cuda(), d_ring, locs, None, out, scratch, scratch.numel())
            ob = out.cpu().numpy()
            qb = q.view(torch.int16).numpy().view(np.uint16)
            for i in range(slots):
                pos = np.arange(t[i] - window, t[i])
                got_rows = view.index_select(0, locs[i, 0].long()).cpu().numpy()
                want_rows = synth.kv_rows_at(w, 9, i, pos).view(np.uint8).reshape(got_rows.shape)
                assert np.array_equal(got_rows, want_rows)
                ref = oracle.mla_attention(qb[i, 0], synth.kv_rows_at(w, 9, i, pos), 576, 512, 576 ** -0.5)
                g = synth.bf16_to_f32(ob[i, 0].view(np.uint16)).astype(np.float64)
                assert np.all(np.abs(g - ref) <= 1e-2 + 2e-2 * np.abs(ref)), f"round {rnd} slot {i}"
            checked += 1
    assert checked >= 2
    log(f"[ring] R_d={ring}: {checked} attention checks over wrapped windows")


@pytest.mark.parametrize("arenas", [0, 2])
def test_promotion_copy_back_after_acceptance(arenas):
    """Verification rounds whose 8-query unions overflow the hot cache into staging (own staging per source,
    and three layers taking turns in two shared arenas): after each layer's attention a random acceptance per
    request promotes the staged rows of committed queries (Adaptive DHiSparse section 3.4, Figure 3 callout 3).
    Checked against the oracle every time, bit for bit: the promoted counts, keys, recency stamps, slot order
    and page table; every hot slot's pool row holds its position's host row afterwards (the copy-back read the
    staging row, no host read); a repeated call promotes nothing; the next round's resolve (promoted rows are
    hits) stays bit-exact with the oracle, and so does the arena's next user."""
    w = synth.WORKLOADS["verify"].scaled(requests=8, layers=3, sources=3, ctx=20_000, queries=8, top_k=512,
                                         hot_slots=1024, staging_rows=8 * 512, seed=3300 + arenas)
    h = Harness(w, steps=4, staging_arenas=arenas)
    rng = np.random.default_rng(77 + arenas)
    R, B = w.requests, w.hot_slots
    total = 0
    for t in range(h.steps):
        for layer in range(w.layers):
            res = h.resolve(layer, t)
            h.check_bytes(res)
            h.attention(layer, t, res, samples=[(0, 0), (5, 3)])
            src = res["src"]
            acc = rng.integers(0, w.queries, size=R).astype(np.int32)
            acc[0] = w.queries - 1                               # everything committed: nothing to move
            d_acc = torch.from_numpy(acc).cuda()
            d_prom = torch.full((R,), -1, dtype=torch.int32, device="cuda")
            h.store.promote_staged(src, res["d_locs"], d_acc, d_prom)
            prom = d_prom.cpu().numpy()
            want = h.ora[src].promote(res["sel"], res["locs"], acc)
            assert np.array_equal(prom, want), f"promoted counts differ: gpu={prom} oracle={want}"
            assert prom[0] == 0
            pool = h.store.pool_rows(src)
            for r in range(R):
                g = h.store.snapshot(src, r)
                a = h.ora[src].snapshot(r)
                for f in ("key", "rec", "order", "pt"):
                    assert np.array_equal(g[f], a[f]), f"{f} differs after promotion r={r}"
                held = np.nonzero(g["key"] >= 0)[0]
                rows = pool.index_select(0, torch.from_numpy(r * B + held).long().cuda()).cpu().numpy()
                assert np.array_equal(rows, h.host_rows(src, r)[g["key"][held]]), f"hot rows differ r={r}"
            total += int(prom.sum())
            h.store.promote_staged(src, res["d_locs"], d_acc, d_prom)
            assert int(d_prom.sum().item()) == 0
            assert np.array_equal(h.ora[src].promote(res["sel"], res["locs"], acc), np.zeros(R, np.int32))
            log(f"[promote arenas={arenas}] step {t} layer {layer}: staged={int(res['stats']['n_staged'].sum())} "
                f"promoted={int(prom.sum())}")
    assert total > 0
    h.close()


def test_promotion_rejects_bad_state():
    st = hsk.KVStore(requests=2, sources=2, row_bytes=1152, hot_slots=8, tail_rows=4, ctx=64, max_queries=2,
                     top_k=4, staging_rows=8)
    locs = torch.zeros((2, 2, 4), dtype=torch.int32, device="cuda")
    acc = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(hsk.HskError) as e:                  # no resolve yet
        st.promote_staged(0, locs, acc)
    assert e.value.status == hsk.HSK_ESTATE
    with pytest.raises(hsk.HskError) as e:
        st.promote_staged(5, locs, acc)
    assert e.value.status == hsk.HSK_EINVAL
    st.close()
