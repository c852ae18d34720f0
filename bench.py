#!/usr/bin/env python3
"""Benchmark: resolve + sparse decode attention, 100K-context batch-64 MLA decode (4 layers) on one GPU.

One step = for each of the 4 layers: hsk_resolve_step (direct pass, hot-cache probe, LRU victims,
metadata update, host->device copies of the distinct misses, all in one kernel) then hsk_sparse_decode_attn (exact MLA
attention of 128 heads over the 2,048 resolved rows) -- the whole hot path, every launch through the
C ABI.  Inputs (host KV rows, selections, queries) are seeded and synthetic (see synth/) and resident
before the timed region; selections are the indexer stand-in (80% kept step to step, Zipf(1.1) fresh
rows).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 63.0
MFMA_BF16_PEAK = 2.5e15
# workgroups (16 waves each) of the copy kernel in the overlapped schedules: 16, 17, 19, 20, 22 and 24 measured
# 0.1-1.8 % slower per 100K batch-64 step than 18
COPY_WORKGROUPS = 18


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def sha_of(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(kernel_key: str, src_path: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get("source_sha") != sha_of(src_path):
        return None
    return e.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(w, sel, q, host_rows_fn, resolve_steps: int, attn_reqs: int, threads: int) -> dict:
    """The oracle on `threads` host threads: resolve of layer 0 for `resolve_steps` steps (all requests,
    OpenMP across requests), then fp64 attention of `attn_reqs` requests at the last of those steps (one
    request per thread at a time; ctypes drops the GIL inside the oracle).  Rows/s of one layer-step."""
    import concurrent.futures as cf

    import oracle
    oracle.set_threads(threads)
    warm = oracle.Source(R=w.requests, ctx=w.ctx, B=w.hot_slots, T=w.tail_rows, row_bytes=w.row_bytes)
    warm.resolve(1, sel[0])      # untimed: starts the OpenMP thread pool
    del warm
    src = oracle.Source(R=w.requests, ctx=w.ctx, B=w.hot_slots, T=w.tail_rows, row_bytes=w.row_bytes)
    src.commit_prefill()
    t0 = time.perf_counter()
    for t in range(resolve_steps):
        src.resolve(t + 1, sel[t])
    t_res = (time.perf_counter() - t0) / resolve_steps
    t = resolve_steps - 1
    reqs = list(range(min(attn_reqs, w.requests)))
    rows = [host_rows_fn(r)[sel[t, r, 0]].view(np.uint16) for r in reqs]

    def one(i):
        return oracle.mla_attention(q[reqs[i], 0], rows[i], w.dk, w.dv, w.scale)

    t0 = time.perf_counter()
    if threads == 1:
        for i in range(len(reqs)):
            one(i)
    else:
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(len(reqs))))
    t_att = (time.perf_counter() - t0) * w.requests / len(reqs)   # scaled to all requests
    per_layer_step = t_res + t_att
    return {"value": w.requests * w.queries * w.top_k / per_layer_step, "unit": "rows/s", "threads": threads,
            "resolve_ms_per_call": t_res * 1e3, "attention_s_per_layer_step": t_att,
            "steps_per_s": 1.0 / (per_layer_step * w.layers)}


def cpu_baseline(w, sel_layer0, q_layer0, host_rows_fn, steps_for_resolve: int, tiny=None) -> dict:
    """The oracle as it stands, on the host's cores, on a bounded sample of the benchmark workload: resolve of
    layer 0 for `steps_for_resolve` steps (all requests) and fp64 attention of every request at the last of
    those steps, on every core available to the process; again on one thread (attention of 8 requests, scaled);
    and the tiny decode (4 requests, 8 steps, all of it) on every core and on one."""
    import oracle
    threads = max(1, len(os.sched_getaffinity(0)))
    full = _oracle_rate(w, sel_layer0, q_layer0, host_rows_fn, steps_for_resolve, w.requests, threads)
    one = _oracle_rate(w, sel_layer0, q_layer0, host_rows_fn, steps_for_resolve, 8, 1)
    out = {"value": full["value"], "unit": "rows/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": (f"{w.name}: layer 0, resolve of all {w.requests} requests for {steps_for_resolve} steps "
                      f"({full['resolve_ms_per_call']:.2f} ms/call on {threads} threads, OpenMP across requests) "
                      f"+ fp64 attention of all {w.requests} requests x {w.heads} heads x {w.top_k} rows at step "
                      f"{steps_for_resolve - 1} ({full['attention_s_per_layer_step']:.2f} s on {threads} threads)"),
           "steps_per_s": full["steps_per_s"],
           "one_thread": {**one, "sample": (f"same resolve sample on 1 thread "
                                            f"({one['resolve_ms_per_call']:.2f} ms/call) + fp64 attention of 8 "
                                            f"requests on 1 thread, scaled to {w.requests}")}}
    if tiny is not None:
        tw, tsel, tq, trows = tiny
        out["tiny_decode"] = {
            "all_threads": _oracle_rate(tw, tsel, tq, trows, tw.steps, tw.requests, threads),
            "one_thread": _oracle_rate(tw, tsel, tq, trows, tw.steps, tw.requests, 1),
            "sample": f"tiny: {tw.requests} requests, {tw.steps} resolve steps, attention of every request "
                      f"at the last step ({tw.heads} heads x {tw.top_k} rows)"}
    oracle.set_threads(threads)
    return out


def tiny_inputs(synth):
    """The tiny decode's inputs for the oracle baseline (host rows generated on the host, no GPU)."""
    tw = synth.WORKLOADS["tiny"]
    sel = synth.selection_stream(tw, 0, steps=tw.steps)
    q = synth.queries(tw, 0, tw.steps - 1)
    rows = {}

    def host_rows(r):
        if r not in rows:
            buf = np.zeros((tw.ctx, tw.row_bytes), np.uint8)
            synth.fill_kv_rows(buf.ctypes.data, tw, 0, r, 0, tw.ctx)
            rows[r] = buf
        return rows[r]
    return tw, sel, q, host_rows


def resolve_algorithmic_bytes(w) -> int:
    """Bytes one resolve call must move for a single-query layer-step with no misses: selections in and
    locations out (4 B each), the slot order (2 B per slot) and keys (4 B per slot) read, the order written,
    one page-table word per selected row and a recency stamp per hit written."""
    R, k, B = w.requests, w.top_k, w.hot_slots
    return R * (k * 4 + k * 4 + B * 2 + B * 4 + B * 2 + k * 4 + k * 4)


def attn_algorithmic_bytes(w) -> int:
    """Selected rows (576 bf16 each), queries, bf16 outputs and locations of one MLA attention call."""
    R, k = w.requests, w.top_k
    return R * k * w.dk * 2 + R * w.heads * w.dk * 2 + R * w.heads * w.dv * 2 + R * k * 4


def hits_only(hsk, w, store, sels, d_q, d_locs, d_stats, ad, scratch, nscratch, pools, first_epoch: int,
              reps: int = 20) -> dict:
    """Every layer repeats its last selection (keep fraction 1): every pending row is a hot hit, so one
    layer-step is resolve (no copies) + attention, bounded by HBM.  The layer-step time comes from `reps`
    back-to-back repetitions of all layers with events only around the whole pass (like the headline step);
    a second pass with events around every call splits it into resolve and attention."""
    import torch
    stream = torch.cuda.current_stream()
    last = [sels[l].shape[0] - 1 for l in range(w.layers)]
    sel_l = [torch.from_numpy(np.ascontiguousarray(sels[l][last[l]])).cuda() for l in range(w.layers)]
    out = torch.empty((w.requests, 1, w.heads, w.dv), dtype=torch.int16, device="cuda")
    e = first_epoch

    def layer_step(l, ev=None):
        if ev is not None:
            ev[0].record(stream)
        store.resolve_step(l, e, sel_l[l], d_locs[l], d_stats[l])
        if ev is not None:
            ev[1].record(stream)
        hsk.sparse_decode_attn(ad, d_q[l][last[l]], pools[l], d_locs[l], None, out, scratch, nscratch)
        if ev is not None:
            ev[2].record(stream)

    for l in range(w.layers):   # the first repetition fetches the repeated rows
        layer_step(l)
    e += 1
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        for l in range(w.layers):
            layer_step(l)
        e += 1
    b.record(stream)
    torch.cuda.synchronize()
    both = a.elapsed_time(b) / (reps * w.layers)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps * w.layers)]
    for i in range(reps):
        for l in range(w.layers):
            layer_step(l, ev[i * w.layers + l])
        e += 1
    torch.cuda.synchronize()
    misses = sum(int(hsk.stats_to_numpy(d_stats[l])["n_miss"].sum()) for l in range(w.layers))
    res_ms = float(np.mean([x.elapsed_time(y) for x, y, _ in ev]))
    att_ms = float(np.mean([y.elapsed_time(z) for _, y, z in ev]))
    nbytes = resolve_algorithmic_bytes(w) + attn_algorithmic_bytes(w)
    gbs = nbytes / (both * 1e-3) / 1e9
    rows = w.requests * w.top_k
    flops = 2.0 * w.heads * (w.dk + w.dv) * rows
    return {"ms_per_layer_step": both, "resolve_ms": res_ms, "attention_ms": att_ms, "misses": misses,
            "algorithmic_bytes_per_layer_step": nbytes, "achieved_GBps": gbs, "hbm_peak_GBps": HBM_PEAK_GBS,
            "frac_hbm": gbs / HBM_PEAK_GBS, "rows_per_s": rows / (both * 1e-3),
            "steps_per_s": 1.0 / (both * 1e-3 * w.layers),
            "resolve_fraction": res_ms / (res_ms + att_ms), "attention_fraction": att_ms / (res_ms + att_ms),
            "attention_TFLOPs": flops / (att_ms * 1e-3) / 1e12,
            "attention_frac_mfma_bf16": flops / (att_ms * 1e-3) / MFMA_BF16_PEAK,
            "note": "ms_per_layer_step from back-to-back layer steps; resolve_ms and attention_ms from HIP events "
                    "around each call (they include the launch gaps the events add)"}


def misses_only(hsk, synth, w, gather_blocks: int, calls: int = 12) -> dict:
    """Fig. 8a analog at the 100K batch-64 shape: B = k, no tail, every call selects k rows no earlier call
    selected, so every selected row is copied from pinned host memory (64 x 2048 x 1152 B = 151 MB)."""
    import torch
    R, k = w.requests, w.top_k
    n = w.ctx
    st = hsk.KVStore(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=k, tail_rows=0, ctx=n, max_queries=1,
                     top_k=k, gather_blocks=gather_blocks)
    for r in range(R):
        synth.fill_kv_rows(st.host_ptr(0, r), w, 0, r, 0, n)
    g = np.random.default_rng([w.seed, 99])
    perms = np.stack([g.permutation(n)[: (calls + 1) * k] for _ in range(R)]).astype(np.int32)
    d_sel = [torch.from_numpy(np.ascontiguousarray(perms[:, c * k:(c + 1) * k].reshape(R, 1, k))).cuda()
             for c in range(calls + 1)]
    locs = torch.empty((R, 1, k), dtype=torch.int32, device="cuda")
    stats = hsk.stats_tensor(R)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    st.resolve_step(0, 1, d_sel[0], locs, stats)  # warm
    fetched = 0
    for c in range(calls):
        ev[c][0].record(stream)
        st.resolve_step(0, c + 2, d_sel[c + 1], locs, stats)
        ev[c][1].record(stream)
    torch.cuda.synchronize()
    fetched = int(hsk.stats_to_numpy(stats)["fetched_bytes"].sum())
    status = st.sync_status()
    st.close()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gbs = fetched / (ms * 1e-3) / 1e9
    return {"bytes_per_call": fetched, "ms_per_call": ms, "achieved_GBps": gbs, "host_link_peak_GBps": PCIE_PEAK_GBS,
            "frac_host_link": gbs / PCIE_PEAK_GBS, "status": status,
            "note": "resolve kernel with its zero-copy miss copies per call; bytes = distinct misses x 1152"}


def misses_sweep(hsk, synth, w, gather_blocks: int, W: int = 8, calls: int = 9) -> dict:
    """Fig. 8a analog with W queries per request: every call selects rows no recent call selected, and the
    W queries of a request share all of their k rows, half of them, or none, so the distinct missing rows per
    request are k, (W + 1) k / 2 or W k.  Each distinct row is copied once (the shared ones dedup); the
    slope of time against copied bytes is the achieved host-link rate.  A fourth point repeats the last
    all-shared call (every row a hot hit, nothing copied): the measured fixed cost of a W-query call.  Each
    mode times `calls` calls after one warm-up call (min, mean and max reported); the fit uses the means."""
    import torch
    R, k, n = w.requests, w.top_k, w.ctx
    S = W * k - k
    st = hsk.KVStore(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=k, tail_rows=0, ctx=n, max_queries=W,
                     top_k=k, staging_rows=S, gather_blocks=gather_blocks)
    for r in range(R):
        synth.fill_kv_rows(st.host_ptr(0, r), w, 0, r, 0, n)
    g = np.random.default_rng([w.seed, 98])
    perms = [g.permutation(n).astype(np.int32) for _ in range(R)]
    cursor = [0] * R

    def take(r, m):
        # fresh positions; the hot cache holds only the last call's k rows, so a position drawn again after
        # a full pass over the context is a miss unless that call selected it (stats count what was copied)
        if cursor[r] + m > n:
            perms[r] = g.permutation(n).astype(np.int32)
            cursor[r] = 0
        a = perms[r][cursor[r]:cursor[r] + m]
        cursor[r] += m
        return a

    locs = torch.empty((R, W, k), dtype=torch.int32, device="cuda")
    stats = hsk.stats_tensor(R)
    stream = torch.cuda.current_stream()
    points, epoch = {}, 1
    last = None
    for mode, shared in (("shared", k), ("half_shared", k // 2), ("disjoint", 0), ("shared_repeat", None)):
        times, byts = [], []
        for c in range(calls + 1):
            if shared is None:
                d = last
            else:
                sel = np.empty((R, W, k), np.int32)
                for r in range(R):
                    common = take(r, shared)
                    for j in range(W):
                        sel[r, j, :shared] = common
                        sel[r, j, shared:] = take(r, k - shared)
                d = torch.from_numpy(sel).cuda()
                if mode == "shared":
                    last = d
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st.resolve_step(0, epoch, d, locs, stats)
            b.record(stream)
            torch.cuda.synchronize()
            epoch += 1
            if c:   # the first call of each mode warms up
                times.append(a.elapsed_time(b))
                byts.append(int(hsk.stats_to_numpy(stats)["fetched_bytes"].sum()))
        points[mode] = {"bytes_per_call": float(np.mean(byts)), "ms_per_call": float(np.mean(times)),
                        "ms_min": float(np.min(times)), "ms_max": float(np.max(times)), "calls": calls}
    status = st.sync_status()
    st.close()
    x = np.array([v["bytes_per_call"] for v in points.values()])
    y = np.array([v["ms_per_call"] for v in points.values()]) * 1e-3
    slope, icpt = np.polyfit(x, y, 1)
    gbs = 1.0 / slope / 1e9
    return {"W": W, "points": points, "fit_GBps": gbs, "fit_intercept_us": icpt * 1e6,
            "zero_copy_call_us": points["shared_repeat"]["ms_per_call"] * 1e3,
            "host_link_peak_GBps": PCIE_PEAK_GBS, "frac_host_link": gbs / PCIE_PEAK_GBS, "status": status,
            "note": f"{R} requests x {W} queries x top-{k}; hot slots = k, staging {S} rows per request; "
                    "call times from HIP events around each call"}


def no_io_bound(hsk, synth, w, sels, d_q, ad, scratch, nscratch, steps: int) -> dict:
    """The no-IO bound (HiSparse section 4.6): layer 0's selection stream resolved by a store whose copies
    from host are skipped (pool rows stale), then attention; timing only, never a correct result."""
    import torch
    R, k = w.requests, w.top_k
    st = hsk.KVStore(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=w.hot_slots, tail_rows=w.tail_rows,
                     ctx=w.ctx, max_queries=1, top_k=k, gather_mode=hsk.GATHER_NO_IO)
    st.commit_prefill()
    locs = torch.empty((R, 1, k), dtype=torch.int32, device="cuda")
    stats = hsk.stats_tensor(R)
    out = torch.empty((R, 1, w.heads, w.dv), dtype=torch.int16, device="cuda")
    pool = st.pool_base(0)
    stream = torch.cuda.current_stream()
    d_sel = [torch.from_numpy(np.ascontiguousarray(sels[0][t])).cuda() for t in range(steps)]
    ev = []
    for t in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        st.resolve_step(0, t + 1, d_sel[t], locs, stats)
        e[1].record(stream)
        hsk.sparse_decode_attn(ad, d_q[0][t], pool, locs, None, out, scratch, nscratch)
        e[2].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    status = st.sync_status()
    st.close()
    ev = ev[2:]
    res = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    both = float(np.mean([a.elapsed_time(c) for a, _, c in ev]))
    return {"ms_per_layer_step": both, "resolve_ms": res, "rows_per_s": R * k / (both * 1e-3),
            "steps_per_s": 1.0 / (both * 1e-3 * w.layers), "status": status,
            "note": "layer 0's selection stream; host copies skipped (pool rows stale)"}


def memcpy_ceiling(nbytes: int = 1 << 28, reps: int = 8) -> dict:
    """Pinned host -> device hipMemcpyAsync of 256 MiB: the DMA-engine ceiling of the host link."""
    import torch
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        d.copy_(h, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return {"bytes": nbytes, "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9}


# ------------------------------------------------------------------------------------------------------
# other workloads (python bench.py --workload verify|adaptive|quest|decode|loadstep): one JSON line each, for the record of
# every hot-path step; the default run is the 100K batch-64 decode above
# ------------------------------------------------------------------------------------------------------
def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def run_verify(hsk, synth, w, steps: int) -> dict:
    """Speculative verification: W queries per request share rows; each distinct missing row is copied once
    and unions beyond the free hot slots go to staging rows (Adaptive DHiSparse section 3.3)."""
    import torch
    R, Q, k, L = w.requests, w.queries, w.top_k, w.layers
    # the layers run one after another, so one staging arena serves them all (Adaptive DHiSparse section 3.4)
    st = hsk.KVStore(requests=R, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                     tail_rows=w.tail_rows, ctx=w.ctx, max_queries=Q, top_k=k, staging_rows=w.staging_rows,
                     staging_arenas=1)
    staging_gib = R * w.staging_rows * w.row_bytes / 2 ** 30
    t0 = time.perf_counter()
    for s_ in range(w.sources):
        for r in range(R):
            synth.fill_kv_rows(st.host_ptr(s_, r), w, s_, r, 0, w.ctx)
    st.commit_prefill()
    log(f"[verify] host rows filled in {time.perf_counter() - t0:.1f} s")
    sels = [torch.from_numpy(synth.selection_stream(w, l, steps=steps)).cuda() for l in range(L)]
    ad = hsk.mla_desc(requests=R, max_queries=Q, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k, row_elems=w.row_elems,
                      scale=w.scale)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q = [torch.from_numpy(synth.queries(w, l, 0).view(np.int16)).cuda() for l in range(L)]
    out = torch.empty((R, Q, w.heads, w.dv), dtype=torch.int16, device="cuda")
    locs = [torch.empty((R, Q, k), dtype=torch.int32, device="cuda") for _ in range(L)]
    stats = [hsk.stats_tensor(R) for _ in range(L)]
    pools = [st.pool_base(l) for l in range(L)]
    res_ms, att_ms, agg = [], [], {"sel": 0, "miss_sel": 0, "miss": 0, "staged": 0}
    stream = torch.cuda.current_stream()
    t_all = 0.0
    for t in range(steps):
        evs = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            e = [_ev() for _ in range(3)]
            e[0].record(stream)
            st.resolve_step(l, t + 1, sels[l][t], locs[l], stats[l])
            e[1].record(stream)
            hsk.sparse_decode_attn(ad, q[l], pools[l], locs[l], None, out, scratch, nb)
            e[2].record(stream)
            evs.append(e)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if t > 0:
            t_all += dt
            for e in evs:
                res_ms.append(e[0].elapsed_time(e[1]))
                att_ms.append(e[1].elapsed_time(e[2]))
            for l in range(L):
                sn = hsk.stats_to_numpy(stats[l])
                agg["sel"] += int(sn["n_sel"].sum()); agg["miss_sel"] += int(sn["n_miss_sel"].sum())
                agg["miss"] += int(sn["n_miss"].sum()); agg["staged"] += int(sn["n_staged"].sum())
    status = st.sync_status()
    st.close()
    ov = _verify_overlapped(hsk, synth, w, steps, sels, q)
    status = status or ov["status"]
    rows = R * Q * k * L * (steps - 1)
    flops = 2.0 * w.heads * (w.dk + w.dv) * R * Q * k
    att = float(np.mean(att_ms))
    ov["rows_per_s"] = rows / (ov["ms_per_step"] * 1e-3 * (steps - 1))
    return {"workload": f"verify: {R} requests x {Q} queries, {L} layers, context {w.ctx}, top-k {k} per query, "
                        f"60% shared, 75% kept, staging {w.staging_rows} rows", "steps_timed": steps - 1,
            "rows_per_s": rows / t_all, "steps_per_s": (steps - 1) / t_all, "resolve_ms": float(np.mean(res_ms)),
            "attention_ms": att, "attention_TFLOPs": flops / (att * 1e-3) / 1e12,
            "attention_frac_mfma_bf16": flops / (att * 1e-3) / 2.5e15,
            "dedup_ratio": agg["miss_sel"] / max(1, agg["miss"]), "fetched_fraction": agg["miss"] / agg["sel"],
            "staged_rows_per_layer_step": agg["staged"] / (L * (steps - 1)),
            "staging_GiB": {"one_shared_arena": staging_gib, "one_arena_per_layer": staging_gib * w.sources},
            "overlapped": ov, "status": status}


def _verify_overlapped(hsk, synth, w, steps: int, sels, q, M: int = 2, fetch_blocks: int = 0) -> dict:
    """The verification step in the overlapped schedule of the headline benchmark: M micro-batches of R/M
    requests, each a deferred store (one shared staging arena, layers in order) on its own stream, one copy
    stream for every fetch, one hsk_resolve_fetch_attend per micro-batch and layer.  Same selections and queries
    as the serial run; steps 1.. are timed (step 0 is cold)."""
    fetch_blocks = fetch_blocks or COPY_WORKGROUPS
    import torch
    R, Q, k, L = w.requests, w.queries, w.top_k, w.layers
    Rm = R // M
    stores, outs, scr, ads, locs, stats = [], [], [], [], [], []
    t0 = time.perf_counter()
    for mb in range(M):
        st = hsk.KVStore(requests=Rm, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                         tail_rows=w.tail_rows, ctx=w.ctx, max_queries=Q, top_k=k, staging_rows=w.staging_rows,
                         staging_arenas=1, gather_mode=hsk.GATHER_DEFERRED, gather_blocks=fetch_blocks)
        for s_ in range(w.sources):
            for r in range(Rm):
                synth.fill_kv_rows(st.host_ptr(s_, r), w, s_, mb * Rm + r, 0, w.ctx)
        st.commit_prefill()
        stores.append(st)
        ad = hsk.mla_desc(requests=Rm, max_queries=Q, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k,
                          row_elems=w.row_elems, scale=w.scale)
        ads.append(ad)
        nb = hsk.attn_scratch_bytes(ad)
        scr.append(torch.empty(nb, dtype=torch.uint8, device="cuda"))
        outs.append(torch.empty((Rm, Q, w.heads, w.dv), dtype=torch.int16, device="cuda"))
        locs.append([torch.empty((Rm, Q, k), dtype=torch.int32, device="cuda") for _ in range(L)])
        stats.append([hsk.stats_tensor(Rm) for _ in range(L)])
    part = [[[sels[l][t][mb * Rm:(mb + 1) * Rm].contiguous() for t in range(steps)] for l in range(L)]
            for mb in range(M)]
    qm = [[q[l][mb * Rm:(mb + 1) * Rm].contiguous() for l in range(L)] for mb in range(M)]
    log(f"[verify] overlapped schedule: {M} micro-batches set up in {time.perf_counter() - t0:.1f} s")
    *streams, copy = hsk.dedicated_streams(M + 1)
    torch.cuda.synchronize()

    def step(t):
        for l in range(L):
            for mb in range(M):
                stores[mb].resolve_fetch_attend(l, t + 1, part[mb][l][t], locs[mb][l], ads[mb], qm[mb][l], outs[mb],
                                                scr[mb], stats=stats[mb][l], stream=streams[mb], copy_stream=copy)

    step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(1, steps):
        step(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    status = 0
    for st in stores:
        status = status or st.sync_status()
        st.close()
    return {"ms_per_step": el * 1e3 / (steps - 1), "micro_batches": M, "requests_per_micro_batch": Rm,
            "fetch_workgroups": fetch_blocks, "status": status}


def run_adaptive(hsk, synth, w, steps: int) -> dict:
    """Load-adaptive residency: optional-history pages resolve directly; a reclaim of whole requests (Eq. 4)
    mid-run drops them and the host-fetch fraction rises (Adaptive DHiSparse section 3.1)."""
    import torch
    R, k, L, P = w.requests, w.top_k, w.layers, w.page_rows
    frac = synth.residency_fractions(w)
    n_pages = w.ctx // P
    page_ids, nxt = [], 0
    for r in range(R):
        ids = np.full(n_pages, -1, np.int32)
        pages = synth.resident_pages(w, r, float(frac[r]))
        ids[pages] = nxt + np.arange(pages.size, dtype=np.int32)
        nxt += pages.size
        page_ids.append(ids)
    st = hsk.KVStore(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=w.hot_slots, tail_rows=w.tail_rows,
                     ctx=w.ctx, page_rows=P, opt_pool_pages=nxt, max_queries=1, top_k=k)
    t0 = time.perf_counter()
    for r in range(R):
        synth.fill_kv_rows(st.host_ptr(0, r), w, 0, r, 0, w.ctx)
    st.commit_prefill()
    for r in range(R):
        st.residency_set(0, r, page_ids[r])
    torch.cuda.synchronize()
    log(f"[adaptive] host rows filled, {nxt} optional pages resident, in {time.perf_counter() - t0:.1f} s")
    sels = [torch.from_numpy(synth.selection_stream(w, l, steps=steps)).cuda() for l in range(L)]
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k, row_elems=w.row_elems,
                      scale=w.scale)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q = [torch.from_numpy(synth.queries(w, l, 0).view(np.int16)).cuda() for l in range(L)]
    out = torch.empty((R, 1, w.heads, w.dv), dtype=torch.int16, device="cuda")
    locs = torch.empty((R, 1, k), dtype=torch.int32, device="cuda")
    stats = hsk.stats_tensor(R)
    pool = st.pool_base(0)
    stream = torch.cuda.current_stream()
    per_step, res_ms, att_ms, t_all = [], [], [], 0.0
    reclaimed = None
    for t in range(steps):
        if t == w.reclaim_step:
            held = np.array([int((ids >= 0).sum()) for ids in page_ids], np.int64)
            holders = np.nonzero(held > 0)[0][:w.reclaim_requests]
            deficit = int(held[holders].sum())
            qn = hsk.reclaim_plan(held, deficit)
            for r in range(qn):
                if held[r] > 0:
                    st.residency_set(0, r, np.full(n_pages, -1, np.int32))
            reclaimed = {"requests_walked": qn, "pages_dropped": deficit}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        miss = sel = opt = 0
        evs = []
        for l in range(L):
            e = [_ev() for _ in range(3)]
            e[0].record(stream)
            st.resolve_step(0, L * t + l + 1, sels[l][t], locs, stats)   # both layers read the one shared source
            e[1].record(stream)
            hsk.sparse_decode_attn(ad, q[l], pool, locs, None, out, scratch, nb)
            e[2].record(stream)
            evs.append(e)
            sn = hsk.stats_to_numpy(stats)
            miss += int(sn["n_miss"].sum()); sel += int(sn["n_sel"].sum()); opt += int(sn["n_opt"].sum())
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if t > 0:
            t_all += dt
            for e in evs:
                res_ms.append(e[0].elapsed_time(e[1]))
                att_ms.append(e[1].elapsed_time(e[2]))
        per_step.append({"step": t, "host_fetch_fraction": miss / sel, "optional_fraction": opt / sel,
                         "ms": dt * 1e3})
    status = st.sync_status()
    st.close()
    before = [x["host_fetch_fraction"] for x in per_step[1:w.reclaim_step]]
    after = [x["host_fetch_fraction"] for x in per_step[w.reclaim_step:]]
    return {"workload": f"adaptive: {R} requests, {L} layers on one shared source, context {w.ctx}, 64-row optional "
                        f"pages at 0/50/100% per request, reclaim of {w.reclaim_requests} requests at step "
                        f"{w.reclaim_step}, top-k {k}", "optional_pages": nxt, "reclaim": reclaimed,
            "rows_per_s": R * k * L * (steps - 1) / t_all, "steps_per_s": (steps - 1) / t_all,
            "resolve_ms": float(np.mean(res_ms)), "attention_ms": float(np.mean(att_ms)),
            "host_fetch_fraction_before_reclaim": float(np.mean(before)),
            "host_fetch_fraction_after_reclaim": float(np.mean(after)), "per_step": per_step, "status": status}


def run_overlapped(hsk, synth, w, sels, q_host, K: int, W: int, M: int, fetch_blocks: int, split: int) -> dict:
    """The benchmark step with the host IO hidden under the other work (HiSparse section 3.5, overlap of IO
    with computation): the batch is served as M micro-batches of R/M requests, each with its own store (in
    HSK_GATHER_DEFERRED mode) and stream, and one copy stream runs every fetch in turn.  Per layer and
    micro-batch, one hsk_resolve_fetch_attend call: resolve (plan only, each request's plan published with the
    call's epoch) on the micro-batch's stream; fetch on the copy stream, its kernel waiting for the published
    plans; event; attention on the micro-batch's stream.  The copies are serialised on the link in issue
    order (micro-batch 0's layer l, then micro-batch 1's, ...), and while the copy stream fetches one
    micro-batch's rows the others resolve and attend; every request still runs its layers in order, each
    layer's attention after its own resolve and fetch.  The fetch kernel's few workgroups leave the other
    compute units to the attention, whose `split` partitions per request (3: 96 workgroups for 32 requests)
    leave room for the fetch and the next resolve.  Same selections and queries as the serial step.

    The M + 1 streams each have a hardware queue of their own (hsk_stream_create): HIP serves ordinary streams
    from a few hardware queues (4 here) handed out in turn, and two of the step's streams on one queue run as one
    FIFO (a fetch then waits behind an attention; the step slows from ~1.7 to ~2.0 ms)."""
    fetch_blocks = fetch_blocks or COPY_WORKGROUPS
    import torch
    R, k = w.requests, w.top_k
    assert R % M == 0
    Rm = R // M
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    stores, d_sel, d_q, d_locs, d_stats, ads, scratch, outs = [], [], [], [], [], [], [], []
    for mb in range(M):
        st = hsk.KVStore(requests=Rm, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                         tail_rows=w.tail_rows, ctx=w.ctx, max_queries=1, top_k=k, gather_blocks=fetch_blocks,
                         gather_mode=hsk.GATHER_DEFERRED)
        for s_ in range(w.sources):
            for r in range(Rm):
                synth.fill_kv_rows(st.host_ptr(s_, r), w, s_, mb * Rm + r, 0, w.ctx)
        st.commit_prefill()
        stores.append(st)
        part = slice(mb * Rm, (mb + 1) * Rm)
        d_sel.append([torch.from_numpy(np.ascontiguousarray(sels[l][:, part])).to(dev) for l in range(w.layers)])
        d_q.append([torch.from_numpy(np.ascontiguousarray(np.stack(q_host[l])[:, part]).view(np.int16)).to(dev)
                    for l in range(w.layers)])
        d_locs.append([torch.empty((Rm, 1, k), dtype=torch.int32, device=dev) for _ in range(w.layers)])
        d_stats.append([hsk.stats_tensor(Rm) for _ in range(w.layers)])
        ad = hsk.mla_desc(requests=Rm, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k,
                          row_elems=w.row_elems, scale=w.scale, split=split)
        ads.append(ad)
        n = hsk.attn_scratch_bytes(ad)
        scratch.append((torch.empty(n, dtype=torch.uint8, device=dev), n))
        outs.append(torch.empty((Rm, 1, w.heads, w.dv), dtype=torch.int16, device=dev))
    log(f"[overlap] {M} micro-batches of {Rm} requests set up in {time.perf_counter() - t0:.1f} s")
    *streams, copy = hsk.dedicated_streams(M + 1)
    torch.cuda.synchronize()

    def step(t):
        for l in range(w.layers):
            for mb in range(M):
                # resolve (plan only) -> fetch on the copy stream -> attention, ordered by the store's events
                stores[mb].resolve_fetch_attend(l, t + 1, d_sel[mb][l][t], d_locs[mb][l], ads[mb], d_q[mb][l][t],
                                                outs[mb], scratch[mb][0], stats=d_stats[mb][l], stream=streams[mb],
                                                copy_stream=copy)

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    misses = [sum(int(hsk.stats_to_numpy(d_stats[mb][l])["n_miss"].sum()) for mb in range(M))
              for l in range(w.layers)]
    status = 0
    for st in stores:
        status = status or st.sync_status()
        st.close()
    return {"ms_per_step": elapsed * 1e3 / K, "steps_per_s": K / elapsed, "micro_batches": M,
            "requests_per_micro_batch": Rm, "fetch_workgroups": fetch_blocks, "attention_partitions": split,
            "distinct_misses_last_step": int(sum(misses)), "status": status}


def run_decode(hsk, synth, w, steps: int) -> dict:
    """The 100K batch-64 shape as a decode loop (HiSparse section 3.3 steps 3-4): per layer, each request
    appends the new token's row (tail ring on the main stream, write-through to host on a backup stream),
    then its selection (which includes the new row) is resolved and attended.  Reports steps/s and the
    append and write-through kernel times beside the resolve and attention calls."""
    import torch
    R, k, L = w.requests, w.top_k, w.layers
    st = hsk.KVStore(requests=R, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                     tail_rows=w.tail_rows, ctx=w.ctx, max_ctx=w.ctx + steps, max_queries=1, top_k=k)
    t0 = time.perf_counter()
    for s_ in range(w.sources):
        for r in range(R):
            synth.fill_kv_rows(st.host_ptr(s_, r), w, s_, r, 0, w.ctx)
    st.commit_prefill()
    log(f"[decode] host rows filled in {time.perf_counter() - t0:.1f} s")
    # selections over the growing context: the stream of the fixed-length run, plus the newest row
    sels = []
    for l in range(L):
        sl = synth.selection_stream(w, l, steps=steps)
        for t in range(steps):
            sl[t, :, 0, 0] = w.ctx + t          # the row appended at step t
        sels.append(torch.from_numpy(sl).cuda())
    rows = [[torch.from_numpy(np.stack([synth.kv_rows(w, l, r, w.ctx + t, 1) for r in range(R)]).view(np.int16))
             .cuda() for t in range(steps)] for l in range(L)]
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k, row_elems=w.row_elems,
                      scale=w.scale)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q = [torch.from_numpy(synth.queries(w, l, 0).view(np.int16)).cuda() for l in range(L)]
    out = torch.empty((R, 1, w.heads, w.dv), dtype=torch.int16, device="cuda")
    locs = torch.empty((R, 1, k), dtype=torch.int32, device="cuda")
    stats = hsk.stats_tensor(R)
    pools = [st.pool_base(l) for l in range(L)]
    main, backup = torch.cuda.current_stream(), torch.cuda.Stream()

    def step(t, evs=None):
        for l in range(L):
            if evs is not None:
                e = [_ev() for _ in range(4)]
                e[0].record(main)
            st.append_rows(l, rows[l][t], 1, stream=main, backup_stream=backup)
            if evs is not None:
                e[1].record(main)
            st.resolve_step(l, t + 1, sels[l][t], locs, stats)
            if evs is not None:
                e[2].record(main)
            hsk.sparse_decode_attn(ad, q[l], pools[l], locs, None, out, scratch, nb)
            if evs is not None:
                e[3].record(main)
                evs.append(e)

    # warm-up, a throughput pass with no events between the calls, then a pass with events
    warm, half = 2, (steps - 2) // 2
    for t in range(warm):
        step(t)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for t in range(warm, warm + half):
        step(t)
    torch.cuda.synchronize()
    t_all = time.perf_counter() - t1
    evs = []
    for t in range(warm + half, steps):
        step(t, evs)
    torch.cuda.synchronize()
    app_ms = [e[0].elapsed_time(e[1]) for e in evs]
    res_ms = [e[1].elapsed_time(e[2]) for e in evs]
    att_ms = [e[2].elapsed_time(e[3]) for e in evs]
    timed = half
    status = st.sync_status()
    tail_ok = all(st.context_rows(l, r) == w.ctx + steps for l in range(L) for r in range(R))
    st.close()
    ov = _decode_overlapped(hsk, synth, w, steps, sels, rows, q, warm, half)
    status = status or ov["status"]
    tail_ok = tail_ok and ov.pop("context_grew")
    return {"workload": f"decode: {R} requests x 1 query, {L} layers with own payloads, context {w.ctx} growing by "
                        f"one row per step, B={w.hot_slots}, tail {w.tail_rows}, top-k {k} (the newest row "
                        f"always selected)", "steps_timed": timed,
            "rows_per_s": R * k * L * timed / t_all, "steps_per_s": timed / t_all,
            "append_call_ms": float(np.mean(app_ms)), "resolve_ms": float(np.mean(res_ms)),
            "attention_ms": float(np.mean(att_ms)), "context_grew": tail_ok, "overlapped": ov, "status": status,
            "note": "append_call_ms covers the tail write on the main stream (event to event); the write-through "
                    "runs on a backup stream beside the following calls"}


def _decode_overlapped(hsk, synth, w, steps: int, sels, rows, q, warm: int, timed: int, M: int = 2,
                       fetch_blocks: int = 0, split: int = 3) -> dict:
    """The decode loop in the overlapped schedule: M micro-batches of R/M requests, each a deferred store on its
    own stream; per layer, the append (tail write and write-through both on the micro-batch's stream: a shared
    backup stream would make each micro-batch's appends wait for the other's, locking them in step) then one
    hsk_resolve_fetch_attend whose fetch runs on the copy stream shared by all.  Same rows, selections and
    queries as the serial loop; the same steps timed."""
    fetch_blocks = fetch_blocks or COPY_WORKGROUPS
    import torch
    R, k, L = w.requests, w.top_k, w.layers
    Rm = R // M
    stores, outs, scr, ads, locs, stats = [], [], [], [], [], []
    for mb in range(M):
        st = hsk.KVStore(requests=Rm, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                         tail_rows=w.tail_rows, ctx=w.ctx, max_ctx=w.ctx + steps, max_queries=1, top_k=k,
                         gather_mode=hsk.GATHER_DEFERRED, gather_blocks=fetch_blocks)
        for s_ in range(w.sources):
            for r in range(Rm):
                synth.fill_kv_rows(st.host_ptr(s_, r), w, s_, mb * Rm + r, 0, w.ctx)
        st.commit_prefill()
        stores.append(st)
        ad = hsk.mla_desc(requests=Rm, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k,
                          row_elems=w.row_elems, scale=w.scale, split=split)
        ads.append(ad)
        scr.append(torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda"))
        outs.append(torch.empty((Rm, 1, w.heads, w.dv), dtype=torch.int16, device="cuda"))
        locs.append(torch.empty((Rm, 1, k), dtype=torch.int32, device="cuda"))
        stats.append(hsk.stats_tensor(Rm))
    part = lambda x, mb: x[mb * Rm:(mb + 1) * Rm].contiguous()  # noqa: E731
    p_sel = [[[part(sels[l][t], mb) for t in range(steps)] for l in range(L)] for mb in range(M)]
    p_rows = [[[part(rows[l][t], mb) for t in range(steps)] for l in range(L)] for mb in range(M)]
    p_q = [[part(q[l], mb) for l in range(L)] for mb in range(M)]
    *streams, copy = hsk.dedicated_streams(M + 1)
    torch.cuda.synchronize()

    def step(t):
        for l in range(L):
            for mb in range(M):
                stores[mb].append_rows(l, p_rows[mb][l][t], 1, stream=streams[mb], backup_stream=streams[mb])
                stores[mb].resolve_fetch_attend(l, t + 1, p_sel[mb][l][t], locs[mb], ads[mb], p_q[mb][l], outs[mb],
                                                scr[mb], stats=stats[mb], stream=streams[mb], copy_stream=copy)

    for t in range(warm):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warm, warm + timed):
        step(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    for t in range(warm + timed, steps):
        step(t)
    torch.cuda.synchronize()
    status = 0
    grew = True
    for st in stores:
        status = status or st.sync_status()
        grew = grew and all(st.context_rows(l, r) == w.ctx + steps for l in range(L) for r in range(Rm))
        st.close()
    return {"ms_per_step": el * 1e3 / timed, "steps_per_s": timed / el, "rows_per_s": R * k * L * timed / el,
            "micro_batches": M, "requests_per_micro_batch": Rm, "fetch_workgroups": fetch_blocks,
            "attention_partitions": split, "context_grew": grew, "status": status}


def _loadstep_arm(hsk, synth, w, ls, optional: bool) -> dict:
    """One arm of the load step: requests arrive in a closed loop at the offered concurrency of each phase,
    are admitted resident-first (their 100K-row history arrives in device memory) when Eq. 3 allows, decode
    their output length (one resolve + MLA attention per step over the admitted slots) and are released; one
    bounded round-robin population attempt per step refills optional history on a copy stream."""
    import collections
    import torch
    R, k, P = w.requests, w.top_k, w.page_rows
    pool_pages = ls.capacity_pages - ls.reserve_pages
    st = hsk.KVStore(requests=R, sources=1, row_bytes=w.row_bytes, hot_slots=w.hot_slots, tail_rows=w.tail_rows,
                     ctx=1, max_ctx=w.ctx, page_rows=P, opt_pool_pages=pool_pages, max_queries=1, top_k=k)
    st.residency_init(ls.capacity_pages, ls.reserve_pages, ls.required_pages, ls.pages_per_attempt, optional)
    hist = torch.from_numpy(synth.kv_rows(w, 0, 0, 0, w.ctx).view(np.int16)).cuda()
    lmax = ls.out_len[1]
    tpl = torch.from_numpy(synth.selection_stream(w, 0, steps=lmax, units=slice(0, ls.templates))).cuda()
    tpl = tpl.reshape(lmax * ls.templates, k)                          # row t * templates + template
    lengths = synth.output_lengths(ls, 1 << 14)
    q = torch.from_numpy(synth.queries(w, 0, 0).view(np.int16)).cuda()
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=k, row_elems=w.row_elems,
                      scale=w.scale)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((R, 1, w.heads, w.dv), dtype=torch.int16, device="cuda")
    locs = torch.empty((R, 1, k), dtype=torch.int32, device="cuda")
    total = sum(n for _, n in ls.phases)
    stats = torch.zeros((total, R * hsk.STATS_BYTES), dtype=torch.uint8, device="cuda")
    pool = st.pool_base(0)
    main, copy = torch.cuda.current_stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    slot_req = [-1] * R              # request in each slot
    slot_t = [0] * R                 # steps it has decoded
    waiting = collections.deque()    # (request, arrival step)
    arrival, admitted_at, finished_at = {}, {}, {}
    next_req, in_system = 0, 0
    ev = [(_ev(), _ev()) for _ in range(total + 1)]
    series, populated = [], []
    t = 0
    for phase, (conc, n_steps) in enumerate(ls.phases):
        for _ in range(n_steps):
            while in_system < conc:                                     # closed loop: arrivals
                waiting.append(next_req)
                arrival[next_req] = t
                next_req += 1
                in_system += 1
            ev[t][0].record(main)
            for _a in range(ls.admit_per_step):                          # admissions, FIFO
                free = [r for r in range(R) if slot_req[r] < 0]
                if not waiting or not free:
                    break
                try:
                    st.admit(free[0], w.ctx, hist, stream=main)
                except hsk.HskError as e:
                    if e.status == hsk.HSK_EWAIT:
                        break
                    raise
                rq = waiting.popleft()
                slot_req[free[0]], slot_t[free[0]] = rq, 0
                admitted_at[rq] = t
            populated.append(st.populate(stream=main, copy_stream=copy) if optional else 0)
            info = st.residency_info()
            ev[t][1].record(main)
            nq = np.array([1 if slot_req[r] >= 0 else 0 for r in range(R)], np.int32)
            idx = np.array([slot_t[r] * ls.templates + (slot_req[r] % ls.templates) if slot_req[r] >= 0 else 0
                            for r in range(R)], np.int64)
            d_nq = torch.from_numpy(nq).cuda()
            sel = tpl.index_select(0, torch.from_numpy(idx).cuda()).reshape(R, 1, k)
            st.resolve_step(0, t + 1, sel, locs, stats[t], nq=d_nq, stream=main)
            hsk.sparse_decode_attn(ad, q, pool, locs, d_nq, out, scratch, nb)
            for r in range(R):                                           # one output step each; finish
                rq = slot_req[r]
                if rq < 0:
                    continue
                slot_t[r] += 1
                if slot_t[r] >= lengths[rq]:
                    st.release(r, stream=main)
                    slot_req[r] = -1
                    finished_at[rq] = t
                    in_system -= 1
            series.append({"step": t, "phase": phase, "admitted": info["admitted"], "waiting": len(waiting),
                           "in_system": in_system,
                           "coverage": info["ready_pages"] / max(1, info["eligible_pages"]),
                           "pending_pages": info["pending_pages"], "unbacked_pages": info["unbacked_pages"]})
            t += 1
    ev[total][0].record(main)
    torch.cuda.synchronize()
    status = st.sync_status()
    sn = stats.cpu().numpy().view(hsk.STATS_DTYPE).reshape(total, R)
    st.close()
    step_ms = [ev[i][0].elapsed_time(ev[i + 1][0]) for i in range(total)]
    decode_ms = [ev[i][1].elapsed_time(ev[i + 1][0]) for i in range(total)]
    admit_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(total)]
    for i, x in enumerate(series):
        sel_i = int(sn["n_sel"][i].sum())
        x["host_share"] = int(sn["n_miss_sel"][i].sum()) / max(1, sel_i)
        x["step_ms"] = step_ms[i]
    phases, t0 = [], 0
    for phase, (conc, n_steps) in enumerate(ls.phases):
        rng_ = range(t0, t0 + n_steps)
        sel_p = int(sn["n_sel"][t0:t0 + n_steps].sum())
        miss_p = int(sn["n_miss_sel"][t0:t0 + n_steps].sum())
        opt_p = int(sn["n_opt"][t0:t0 + n_steps].sum())
        adm = [rq for rq, a in admitted_at.items() if a in rng_]
        fin = [rq for rq, f in finished_at.items() if f in rng_]
        full = next((i - t0 for i in rng_ if series[i]["admitted"] >= R), None)
        half = next((i - t0 for i in rng_ if series[i]["coverage"] > 0.5), None)
        # the steps after the in-flight count came back to the offered load (the last row of Table A1)
        settled = [i for i in rng_ if series[i]["in_system"] <= conc]
        sel_s = int(sn["n_sel"][settled].sum()) if settled else 0
        miss_s = int(sn["n_miss_sel"][settled].sum()) if settled else 0
        phases.append({"offered": conc, "steps": n_steps, "requests_admitted": len(adm), "requests_finished": len(fin),
                       "host_fetched_pct": 100.0 * miss_p / max(1, sel_p), "optional_pct": 100.0 * opt_p / max(1, sel_p),
                       "mean_coverage": float(np.mean([series[i]["coverage"] for i in rng_])),
                       "decode_ms_per_step": float(np.mean([decode_ms[i] for i in rng_])),
                       "step_ms": float(np.mean([step_ms[i] for i in rng_])),
                       "admission_ms_per_step": float(np.mean([admit_ms[i] for i in rng_])),
                       "alloc_wait_steps": float(np.mean([admitted_at[rq] - arrival[rq] for rq in adm])) if adm else None,
                       "steps_to_fill_slots": full, "steps_to_coverage_50pct": half,
                       "pages_populated": int(sum(populated[t0:t0 + n_steps])),
                       "settled_steps": len(settled),
                       "host_fetched_pct_settled": 100.0 * miss_s / sel_s if sel_s else None,
                       "step_ms_settled": float(np.mean([step_ms[i] for i in settled])) if settled else None})
        t0 += n_steps
    return {"status": status, "phases": phases, "series": series[::5]}


def run_loadstep(hsk, synth, w, steps: int) -> dict:
    """Adaptive DHiSparse 4.3.1 (Figure 6, Table A1 shape): the load step replayed on the kernels, optional
    residency on and off; coverage, host-fetched share and step time per phase."""
    ls = synth.LOADSTEP
    arms = {}
    for optional in (True, False):
        t0 = time.perf_counter()
        arms["residency_on" if optional else "residency_off"] = _loadstep_arm(hsk, synth, w, ls, optional)
        log(f"[loadstep] arm optional={optional} in {time.perf_counter() - t0:.1f} s")
    return {"workload": f"load step, one GPU's share: {w.requests} slots, offered concurrency "
                        f"{' -> '.join(str(c) for c, _ in ls.phases)} for {ls.phases[0][1]} steps each, imported "
                        f"history {w.ctx} rows in {w.page_rows}-row pages (resident-first admission), output "
                        f"{ls.out_len[0]}-{ls.out_len[1]} steps, B={w.hot_slots}, T={w.tail_rows}, top-k {w.top_k}, "
                        f"{w.heads} heads; capacity {ls.capacity_pages} pages, {ls.required_pages} required per "
                        f"request, reserve {ls.reserve_pages}, {ls.pages_per_attempt} pages per population attempt, "
                        f"{ls.admit_per_step} admissions per step", **arms}


def run_quest(hsk, synth, w, steps: int) -> dict:
    """Page-level GQA: layer 0 resolves the shared page selection; layers 1..7 replay its miss plan on a side
    stream while the previous layer's attention runs (HiSparse section 3.5)."""
    import torch
    U, k, L = w.units, w.top_k, w.layers
    st = hsk.KVStore(requests=U, sources=L, row_bytes=w.row_bytes, hot_slots=w.hot_slots, tail_rows=0, ctx=w.ctx,
                     max_queries=1, top_k=k, host_alias=True)
    t0 = time.perf_counter()
    for u in range(U):
        synth.fill_kv_rows(st.host_ptr(0, u), w, 0, u, 0, w.ctx)
    log(f"[quest] host pages filled in {time.perf_counter() - t0:.1f} s")
    sel = torch.from_numpy(synth.selection_stream(w, 0, steps=steps)).cuda()
    ad = hsk.gqa_desc(requests=w.requests, heads=w.heads, kv_heads=w.kv_heads, dh=w.dk, top_k=k,
                      page_tokens=w.page_tokens, scale=w.scale)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q = [torch.from_numpy(synth.queries(w, l, 0).view(np.int16)).cuda() for l in range(L)]
    out = torch.empty((w.requests, w.heads, w.dk), dtype=torch.int16, device="cuda")
    locs = torch.empty((U, 1, k), dtype=torch.int32, device="cuda")
    stats = hsk.stats_tensor(U)
    pools = [st.pool_base(l) for l in range(L)]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()

    def step(t, overlap: bool, evs=None):
        st.resolve_step(0, t + 1, sel[t], locs, stats)
        if evs is not None:
            evs["res"][1].record(main)
        done = []
        if overlap:
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
            for l in range(1, L):
                st.replay_plan(0, l, stream=side)
                e = torch.cuda.Event()
                e.record(side)
                done.append(e)
        for l in range(L):
            if l and overlap:
                main.wait_event(done[l - 1])
            elif l:
                st.replay_plan(0, l, stream=main)
            if evs is not None:
                evs["att"][l][0].record(main)
            hsk.sparse_decode_attn(ad, q[l], pools[l], locs, None, out, scratch, nb)
            if evs is not None:
                evs["att"][l][1].record(main)

    res = {}
    for mode, overlap in (("sequential", False), ("side_stream", True)):
        tt, att = 0.0, []
        for t in range(steps):
            evs = {"res": [_ev(), _ev()], "att": [[_ev(), _ev()] for _ in range(L)]}
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            evs["res"][0].record(main)
            step(t, overlap, evs)
            torch.cuda.synchronize()
            if t > 0:
                tt += time.perf_counter() - t0
                att += [a.elapsed_time(b) for a, b in evs["att"]]
        res[mode] = {"ms_per_step": tt * 1e3 / (steps - 1), "gqa_attention_ms": float(np.mean(att))}
        if mode == "sequential":
            st.close()
            st = hsk.KVStore(requests=U, sources=L, row_bytes=w.row_bytes, hot_slots=w.hot_slots, tail_rows=0,
                             ctx=w.ctx, max_queries=1, top_k=k, host_alias=True)
            for u in range(U):
                synth.fill_kv_rows(st.host_ptr(0, u), w, 0, u, 0, w.ctx)
            pools = [st.pool_base(l) for l in range(L)]
    misses = int(hsk.stats_to_numpy(stats)["n_miss"].sum())
    status = st.sync_status()
    st.close()
    att = res["sequential"]["gqa_attention_ms"]  # on one stream the events bracket the kernels alone
    nbytes = U * k * w.row_bytes + w.requests * w.heads * w.dk * 2 * 2 + U * k * 4
    return {"workload": f"quest: {w.requests} requests x {w.kv_heads} KV heads, {L} layers, {w.ctx} pages of "
                        f"{w.page_tokens} tokens, top-{k} pages shared by all layers, {w.hot_slots} page slots",
            "note": "layers 1..7 read layer 0's host payload (one 17 GB host copy instead of 137 GB); the bytes "
                    "moved per layer are the same", "modes": res,
            "overlap_gain": res["sequential"]["ms_per_step"] / res["side_stream"]["ms_per_step"],
            "gqa_algorithmic_bytes_per_layer": nbytes, "gqa_achieved_GBps": nbytes / (att * 1e-3) / 1e9,
            "gqa_frac_hbm": nbytes / (att * 1e-3) / 1e9 / HBM_PEAK_GBS, "last_step_misses": misses,
            "status": status}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the hits-only, misses-only and memcpy runs")
    ap.add_argument("--workload", default="dsa100k",
                    choices=["dsa100k", "verify", "adaptive", "quest", "decode", "loadstep"])
    ap.add_argument("--gather-blocks", type=int, default=0,
                    help="workgroups of the plan-replay copy kernel (0 = automatic); resolve calls copy their "
                         "misses inside the resolve kernel")
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--micro-batches", type=int, default=2,
                    help="the headline step: 1 = one store, each layer's resolve (with its copies) then attention "
                         "on one stream; M > 1 = M micro-batches with the copies on a copy stream under the "
                         "other micro-batches' work (the serial step is reported beside it)")
    ap.add_argument("--only", choices=["hits", "sweep"], default=None,
                    help="profiling aid: after the warmup steps run only the hits-only layer steps or the W = 8 "
                         "miss sweep, and print their result")
    ap.add_argument("--fetch-blocks", type=int, default=0,
                    help="workgroups (16 waves each) of the copy kernel in the overlapped step (0: COPY_WORKGROUPS)")
    ap.add_argument("--overlap-split", type=int, default=3,
                    help="attention partitions per request in the overlapped step")
    ap.add_argument("--path", default="separate", choices=["separate", "fused"],
                    help="separate: hsk_resolve_step then hsk_sparse_decode_attn per layer; fused: "
                         "hsk_resolve_attend per layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 4 device-to-device copies of 1 GiB (the known-size kernel that scales the "
                         "HBM byte counters of a profile)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs the hot path on a single MI355X and has no "
              "multi-GPU path (--gpus must be 1)", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 4}))
        return 0

    import hierarchical_sparse_kv_layer_amd as hsk
    import synth

    w = synth.WORKLOADS["dsa100k" if args.workload == "decode" else args.workload]
    if args.workload != "dsa100k":
        torch.cuda.set_device(0)
        fn = {"verify": run_verify, "adaptive": run_adaptive, "quest": run_quest, "decode": run_decode,
              "loadstep": run_loadstep}[args.workload]
        steps = args.steps if args.steps != 32 else w.steps
        r = fn(hsk, synth, w, steps)
        hsk.release_dedicated_streams()
        print(json.dumps(r), flush=True)
        return 0
    assert w.kind == "mla" and w.queries == 1, "the benchmark line is the single-query MLA decode"
    K, W = args.steps, args.warmup
    total_steps = W + K + min(K, 16)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    store = hsk.KVStore(requests=w.requests, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                        tail_rows=w.tail_rows, ctx=w.ctx, max_queries=1, top_k=w.top_k,
                        gather_blocks=args.gather_blocks)
    for s in range(w.sources):
        for r in range(w.requests):
            synth.fill_kv_rows(store.host_ptr(s, r), w, s, r, 0, w.ctx)
    store.commit_prefill()
    log(f"[bench] host rows filled and tails committed in {time.perf_counter() - t_setup:.1f} s")
    sels = [synth.selection_stream(w, l, steps=total_steps) for l in range(w.layers)]
    d_sel = [torch.from_numpy(s).to(dev) for s in sels]                      # [steps][R][1][k] per layer
    q_host = [[synth.queries(w, l, t) for t in range(total_steps)] for l in range(w.layers)]
    d_q = [torch.from_numpy(np.stack(q_host[l]).view(np.int16)).to(dev) for l in range(w.layers)]
    d_locs = [torch.empty((w.requests, 1, w.top_k), dtype=torch.int32, device=dev) for _ in range(w.layers)]
    d_stats = [hsk.stats_tensor(w.requests) for _ in range(w.layers)]
    ad = hsk.mla_desc(requests=w.requests, max_queries=1, heads=w.heads, dk=w.dk, dv=w.dv, top_k=w.top_k,
                      row_elems=w.row_elems, scale=w.scale, split=args.split)
    nscratch = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nscratch, dtype=torch.uint8, device=dev)
    out = torch.empty((w.requests, 1, w.heads, w.dv), dtype=torch.int16, device=dev)
    pools = [store.pool_base(l) for l in range(w.layers)]
    stream = torch.cuda.current_stream()
    log(f"[bench] inputs resident ({time.perf_counter() - t_setup:.1f} s); warmup {W} steps")

    fused = args.path == "fused"

    def run_step(t, ev=None):
        for l in range(w.layers):
            if ev is not None:
                ev[l][0].record(stream)
            if fused:
                store.resolve_attend(l, t + 1, d_sel[l][t], d_locs[l], ad, d_q[l][t], out, scratch,
                                     stats=d_stats[l])
                if ev is not None:
                    ev[l][1].record(stream)
            else:
                store.resolve_step(l, t + 1, d_sel[l][t], d_locs[l], d_stats[l])
                if ev is not None:
                    ev[l][1].record(stream)
                hsk.sparse_decode_attn(ad, d_q[l][t], pools[l], d_locs[l], None, out, scratch, nscratch)
            if ev is not None:
                ev[l][2].record(stream)

    for t in range(W):
        run_step(t)
    torch.cuda.synchronize()
    if store.sync_status() != 0:
        log("[bench] device-side error during warmup")
        return 1
    if args.only:
        if args.only == "hits":
            r = hits_only(hsk, w, store, sels, d_q, d_locs, d_stats, ad, scratch, nscratch, pools, first_epoch=W + 1)
        else:
            r = misses_sweep(hsk, synth, w, args.gather_blocks)
        print(json.dumps({args.only: r}), flush=True)
        store.close()
        return 0
    misses = []
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run_step(W + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-call durations on the launch stream, from HIP events, over K more steps (events between the calls
    # would add small gaps to the throughput pass above)
    KE = min(K, 16)
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(w.layers)] for _ in range(KE)]
    for i in range(KE):
        run_step(W + K + i, events[i])
    torch.cuda.synchronize()
    status = store.sync_status()
    res_ms, att_ms = [], []
    for i in range(KE):
        for l in range(w.layers):
            a, b, c = events[i][l]
            res_ms.append(a.elapsed_time(b))
            att_ms.append(b.elapsed_time(c))
    for l in range(w.layers):
        st = hsk.stats_to_numpy(d_stats[l])
        misses.append(int(st["n_miss"].sum()))
    rows_per_step = w.requests * w.queries * w.top_k * w.layers
    value = rows_per_step * K / elapsed
    ms_per_step = elapsed * 1e3 / K
    att_avg = float(np.mean(att_ms))
    res_avg = float(np.mean(res_ms))
    attn_bytes = attn_algorithmic_bytes(w)
    achieved = attn_bytes / (att_avg * 1e-3) / 1e9
    traffic = counter_traffic("mla_attention_call", os.path.join(ROOT, "hierarchical_sparse_kv_layer_amd", "csrc",
                                                                 "attention.hip"))
    result = {
        "metric": "selected KV rows resolved+attended/s; decode steps/s at 100K ctx, batch 64",
        "value": value, "unit": "rows/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.requests} requests x 1 query, {w.layers} layers with own payloads, "
                               f"context {w.ctx}, B={w.hot_slots}, tail {w.tail_rows}, top-k {w.top_k}, "
                               f"{w.heads} heads, dk {w.dk}, dv {w.dv}, 80% kept + Zipf(1.1)",
                   "global_batch": w.requests, "seq_len": w.ctx, "parallelism": "none (1 GPU)",
                   "path": args.path},
        "steps_per_s": K / elapsed,
        "roofline": {"bound": "hbm", "kernel": "hsk_sparse_decode_attn call (mla32_kernel + combine_kernel)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": attn_bytes,
                     "avg_launch_ms": att_avg},
        "resolve": {"avg_call_ms": res_avg, "avg_distinct_misses_per_layer_step": float(np.mean(misses)),
                    "fetched_bytes_per_call": float(np.mean(misses)) * w.row_bytes,
                    "host_link_GBps_lower_bound": float(np.mean(misses)) * w.row_bytes / (res_avg * 1e-3) / 1e9,
                    "host_link_peak_GBps": PCIE_PEAK_GBS},
        "status": status,
    }
    if args.micro_batches > 1 and not fused:
        # the headline step: the same selections and queries, with the copies under the other work
        ov = run_overlapped(hsk, synth, w, sels, q_host, K, W, args.micro_batches, args.fetch_blocks,
                            args.overlap_split)
        result["serial"] = {"value": value, "ms_per_step": ms_per_step, "steps_per_s": K / elapsed,
                            "schedule": "one store; per layer hsk_resolve_step (copies inside) then "
                                        "hsk_sparse_decode_attn, one stream"}
        result["overlap"] = ov
        result["value"] = rows_per_step * ov["steps_per_s"]
        result["ms_per_step"] = ov["ms_per_step"]
        result["steps_per_s"] = ov["steps_per_s"]
        result["config"]["schedule"] = (f"{ov['micro_batches']} micro-batches of {ov['requests_per_micro_batch']} "
                                        f"requests, one stream each; hsk_fetch_plan on a copy stream "
                                        f"({ov['fetch_workgroups']} copy workgroups); attention in "
                                        f"{ov['attention_partitions']} partitions per request")
        result["status"] = status = status or ov["status"]
    else:
        result["config"]["schedule"] = "one store, one stream"
    if not args.no_extras:
        result["hits_only"] = hits_only(hsk, w, store, sels, d_q, d_locs, d_stats, ad, scratch, nscratch, pools,
                                        first_epoch=total_steps + 1)
        result["misses_only"] = misses_only(hsk, synth, w, args.gather_blocks)
        result["misses_sweep_w8"] = misses_sweep(hsk, synth, w, args.gather_blocks)
        result["no_io_bound"] = no_io_bound(hsk, synth, w, sels, d_q, ad, scratch, nscratch,
                                            steps=min(total_steps, 12))
        result["host_link_ceiling"] = memcpy_ceiling()
    # the overlapped schedule's streams: nothing was allocated on them, so they can go before the process ends
    hsk.release_dedicated_streams()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline(w, sels[0], q_host[0][min(3, total_steps) - 1],
                                              lambda r: store.host_rows(0, r), min(4, total_steps),
                                              tiny=tiny_inputs(synth))
    print(json.dumps(result), flush=True)
    store.close()
    return 0 if status == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
