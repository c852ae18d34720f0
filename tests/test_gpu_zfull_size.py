"""GPU parity at the benchmark's full sizes, in the launch configurations the benchmark times, for the
workloads whose other parity tests run scaled down: speculative verification (128 requests x 16 queries:
2,048 queries, one attention partition), page-level GQA with plan replay (32 requests x 8 KV heads = 256
units) and load-adaptive residency (64 requests, 500,000-row context, reclaim of 16 requests); and the
100K-context batch-64 decode in the benchmark's overlapped schedule (two micro-batches of 32 requests).

Resolution is compared bit-exactly on every call (locations, statistics, miss plan; slot metadata on a
subset of requests); pool bytes and attention on sampled requests.  Attention within
|gpu - ref| <= 1e-2 + 2e-2 |ref| of the fp64 oracle.  Each test prints its case before the GPU work.
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
from hsk_harness import Harness, log  # noqa: E402


def test_verify_full_size_launch_sampled():
    """One layer of the verification workload at full size: 128 requests x 16 queries x top-2048, 60 %
    shared rows, staging 32,768 rows per request; attention over all 2,048 queries in one launch."""
    w = synth.WORKLOADS["verify"].scaled(layers=1, sources=1)
    log(f"[full verify] R={w.requests} Q={w.queries} k={w.top_k} ctx={w.ctx}")
    h = Harness(w, steps=2)
    rng = np.random.default_rng(17)
    for t in range(h.steps):
        res = h.resolve(0, t, meta_reqs=range(0, w.requests, 37))
        reqs = [int(r) for r in rng.choice(w.requests, size=3, replace=False)]
        h.check_bytes(res, reqs=reqs)
        samples = [(r, int(j)) for r in reqs for j in rng.choice(w.queries, size=2, replace=False)]
        err = h.attention(0, t, res, samples=samples)
        st = res["stats"]
        log(f"[full verify] step {t}: miss_sel={int(st['n_miss_sel'].sum())} distinct={int(st['n_miss'].sum())} "
            f"staged={int(st['n_staged'].sum())} attn err {err[0]:.2e}")
    h.close()


def test_quest_full_size_overlapped_layer():
    """Page-level GQA at full size through hsk_resolve_fetch_attend on a deferred store: 256 units, top 256 of
    8,192 pages, the layer-0 resolve, its fetch on a copy stream and the page attention in one call; then layer
    1's replay of the plan, which copies in deferred stores too.  Resolution bit-exact, pool bytes and attention
    sampled."""
    w = synth.WORKLOADS["quest"]
    log(f"[full quest overlap] R={w.requests} Hkv={w.kv_heads} k={w.top_k} pages={w.ctx}")
    h = Harness(w, steps=2, deferred=True)
    rng = np.random.default_rng(29)
    for t in range(h.steps):
        res = h.resolve(0, t, overlap=True, meta_reqs=range(0, h.U, 51))
        units = [int(u) for u in rng.choice(h.U, size=4, replace=False)]
        h.check_bytes(res, source=0, reqs=units)
        err = h.check_attention(0, t, res, res["out"], samples=units, source=0)
        if t == 0:
            h.store.replay_plan(0, 1)
            h.check_bytes(res, source=1, reqs=units)
        log(f"[full quest overlap] step {t}: misses={int(res['stats']['n_miss'].sum())} attn err {err[0]:.2e}")
    h.close()


def test_quest_full_size_replay_sampled():
    """Page-level GQA at full size: 256 (request, KV head) units, top 256 of 8,192 pages, layer 0 resolves
    and layers 1-7 replay its miss plan on a side stream; every layer's attention sampled."""
    w = synth.WORKLOADS["quest"]
    log(f"[full quest] R={w.requests} Hkv={w.kv_heads} k={w.top_k} pages={w.ctx} layers={w.layers}")
    h = Harness(w, steps=2)
    rng = np.random.default_rng(23)
    side = torch.cuda.Stream()
    for t in range(h.steps):
        res = h.resolve(0, t, meta_reqs=range(0, h.U, 51))
        h.check_bytes(res, source=0, reqs=[int(u) for u in rng.choice(h.U, size=4, replace=False)])
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
        worst = 0.0
        for layer in range(w.layers):
            if layer:
                torch.cuda.current_stream().wait_event(done[layer - 1])
            units = [int(u) for u in rng.choice(h.U, size=3, replace=False)]
            err = h.attention(layer, t, res, samples=units, source=layer)
            worst = max(worst, err[0])
            if layer == w.layers - 1:
                h.check_bytes(res, source=layer, reqs=units)
        log(f"[full quest] step {t}: misses={int(res['stats']['n_miss'].sum())} worst attn err {worst:.2e}")
    h.close()


def test_adaptive_full_size_reclaim_sampled():
    """Load-adaptive residency at full size: 64 requests with 500,000-row histories on one shared source
    read by two layers, optional pages seeded at 0 / 50 / 100 %, a reclaim of 16 requests at step 1."""
    w = synth.WORKLOADS["adaptive"].scaled(steps=3, reclaim_step=1)
    log(f"[full adaptive] R={w.requests} ctx={w.ctx} layers={w.layers} reclaim {w.reclaim_requests} at step 1")
    h = Harness(w, steps=w.steps)
    rng = np.random.default_rng(29)
    for t in range(h.steps):
        if t == w.reclaim_step:
            h.reclaim()
        tot_miss = tot_sel = 0
        for layer in range(w.layers):
            res = h.resolve(layer, t, meta_reqs=range(0, w.requests, 21))
            reqs = [int(r) for r in rng.choice(w.requests, size=2, replace=False)]
            h.check_bytes(res, reqs=reqs)
            h.attention(layer, t, res, samples=[(r, 0) for r in reqs])
            tot_miss += int(res["stats"]["n_miss"].sum())
            tot_sel += int(res["stats"]["n_sel"].sum())
        log(f"[full adaptive] step {t}: host-fetch fraction {tot_miss / tot_sel:.4f}")
    h.close()


def test_dsa100k_overlapped_schedule_full_size():
    """The benchmark's overlapped step at full size: two micro-batches of 32 requests (deferred stores, 4 layers
    with their own payloads, 100,000-row contexts), each on its own stream, one copy stream shared by both (all
    three on hardware queues of their own, hsk_stream_create), 18 copy workgroups, attention in 3 partitions
    per request, all calls of a step queued before any check.
    Every call's locations and statistics against the oracle, bit for bit; pool bytes and attention sampled."""
    base = synth.WORKLOADS["dsa100k"]
    M, Rm = 2, base.requests // 2
    ws = [base.scaled(requests=Rm, seed=base.seed + 100 * mb) for mb in range(M)]
    log(f"[full overlap] {M} micro-batches x {Rm} requests, {base.layers} layers, ctx={base.ctx}")
    hs = [Harness(w, steps=2, gather_blocks=18, check_meta_every=2, deferred=True) for w in ws]
    *streams, copy = hsk.dedicated_streams(M + 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(23)
    for t in range(hs[0].steps):
        # every input of the step first (on the default stream), then all calls queued without a host wait, in the
        # benchmark's order: layer by layer, micro-batch 0 then 1
        calls = []
        for layer in range(base.layers):
            for mb, (h, w) in enumerate(zip(hs, ws)):
                sel = h.sel[layer][t]
                d_sel = torch.from_numpy(sel).cuda()
                ad = hsk.mla_desc(requests=Rm, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=w.top_k,
                                  row_elems=w.row_elems, scale=w.scale, split=3)
                calls.append(dict(mb=mb, layer=layer, sel=sel, d_sel=d_sel, d_locs=torch.full_like(d_sel, -7),
                                  d_stats=hsk.stats_tensor(Rm), ad=ad,
                                  q=torch.from_numpy(synth.queries(w, layer, t).view(np.int16)).cuda(),
                                  out=torch.zeros((Rm, 1, w.heads, w.dv), dtype=torch.int16, device="cuda"),
                                  scratch=torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda")))
        torch.cuda.synchronize()
        for c in calls:
            h = hs[c["mb"]]
            h.store.resolve_fetch_attend(h.source_of(c["layer"]), h.epoch_of(c["layer"], t), c["d_sel"], c["d_locs"],
                                         c["ad"], c["q"], c["out"], c["scratch"], stats=c["d_stats"],
                                         stream=streams[c["mb"]], copy_stream=copy)
        torch.cuda.synchronize()
        for c in calls:
            mb, layer, sel, d_locs, d_stats, out = c["mb"], c["layer"], c["sel"], c["d_locs"], c["d_stats"], c["out"]
            h, w = hs[mb], ws[mb]
            src = h.source_of(layer)
            assert h.store.sync_status() == 0
            o = h.ora[src].resolve(h.epoch_of(layer, t), sel)
            locs = d_locs.cpu().numpy()
            assert np.array_equal(locs, o["locs"]), (mb, layer, t)
            st = hsk.stats_to_numpy(d_stats)
            for f in oracle.STATS_DTYPE.names:
                if f != "pad":
                    assert np.array_equal(st[f], o["stats"][f]), (mb, layer, t, f)
            reqs = [int(r) for r in rng.choice(Rm, size=2, replace=False)]
            res = {"sel": sel, "d_locs": d_locs, "src": src}
            h.check_bytes(res, reqs=reqs)
            err = h.check_attention(layer, t, res, out, samples=[(r, 0) for r in reqs])
            log(f"[full overlap] step {t} layer {layer} micro-batch {mb}: miss={int(st['n_miss'].sum())} "
                f"attn err {err[0]:.2e}")
    for h in hs:
        h.close()
