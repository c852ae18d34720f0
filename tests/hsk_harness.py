"""Runs one workload through the HIP path (libhsk.so via the Python binding) and the CPU oracle side by
side, on the same seeded inputs, and compares them.  Used by the GPU parity tests only.

Comparisons per resolve call (bit-exact): every location, every stats field, the miss plan (distinct
missing positions in miss order and the pool row each went to), and for chosen requests the hot-cache
metadata (keys, recency stamps, slot order, page table).  Exactness (Adaptive DHiSparse Eq. 12): the
pool bytes at every emitted location equal the host bytes of the selected row.  Attention: GPU bf16
output against the oracle's fp64 result within |gpu - ref| <= 1e-2 + 2e-2 |ref| per element.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import hierarchical_sparse_kv_layer_amd as hsk
import oracle
import synth

ATOL, RTOL = 1e-2, 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Harness:
    def __init__(self, w: synth.Workload, steps: int | None = None, gather_blocks: int = 0, check_meta_every: int = 1,
                 staging_arenas: int = 0, deferred: bool = False):
        """deferred: the store plans only (HSK_GATHER_DEFERRED) and each resolve is followed by hsk_fetch_plan
        on a side stream, ordered by events (resolve -> fetch -> readers)."""
        self.w = w
        self.deferred = deferred
        self.copy_stream = torch.cuda.Stream() if deferred else None
        self.steps = w.steps if steps is None else steps
        self.U = w.units
        self.check_meta_every = check_meta_every
        self.page_rows = w.page_rows if w.residency_levels else 0
        self.frac = synth.residency_fractions(w)
        self.page_ids = []
        opt_pages = 0
        if self.page_rows:
            n_pages = w.ctx // self.page_rows
            for r in range(self.U):
                ids = np.full(n_pages, -1, np.int32)
                pages = synth.resident_pages(w, r, float(self.frac[r]))
                ids[pages] = opt_pages + np.arange(pages.size, dtype=np.int32)
                opt_pages += pages.size
                self.page_ids.append(ids)
        self.opt_pool_pages = opt_pages
        log(f"[harness] {w.name}: units={self.U} sources={w.sources} ctx={w.ctx} B={w.hot_slots} k={w.top_k} "
            f"Q={w.queries} steps={self.steps} opt_pages={opt_pages}")
        self.store = hsk.KVStore(requests=self.U, sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
                                 tail_rows=w.tail_rows, ctx=w.ctx, page_rows=self.page_rows,
                                 opt_pool_pages=opt_pages, max_queries=w.queries, top_k=w.top_k,
                                 staging_rows=w.staging_rows, host_alias=w.host_alias, gather_blocks=gather_blocks,
                                 staging_arenas=staging_arenas,
                                 gather_mode=hsk.GATHER_DEFERRED if deferred else hsk.GATHER_ZEROCOPY)
        host_sources = 1 if w.host_alias else w.sources
        for s in range(host_sources):
            for r in range(self.U):
                synth.fill_kv_rows(self.store.host_ptr(s, r), w, s, r, 0, w.ctx)
        self.store.commit_prefill()
        # metadata-carrying sources: one per payload source, except that shared-selection layers replay
        # their anchor's plan and carry no state of their own
        self.meta_sources = [0] if w.shared_selection else list(range(w.sources))
        # with shared staging arenas, source s stages into arena s mod A after the last source region
        P = self.store.rows_per_source

        def stg_base(s):
            return w.sources * P + (s % staging_arenas) * self.U * w.staging_rows - s * P if staging_arenas else -1
        self.ora = {s: oracle.Source(R=self.U, ctx=w.ctx, B=w.hot_slots, T=w.tail_rows, page_rows=self.page_rows,
                                     opt_pool_pages=opt_pages, staging_rows=w.staging_rows, row_bytes=w.row_bytes,
                                     stg_base=stg_base(s))
                    for s in self.meta_sources}
        for o in self.ora.values():
            o.commit_prefill()
        if self.page_rows:
            for r in range(self.U):
                self.store.residency_set(0, r, self.page_ids[r])
                assert self.ora[0].residency_set(r, self.page_ids[r]) == 0
        torch.cuda.synchronize()
        self.sel = {}
        sel_layers = [0] if w.shared_selection else list(range(w.layers))
        for l in sel_layers:
            self.sel[l] = synth.selection_stream(w, l, steps=self.steps)
        self.host_fetch = []

    # ------------------------------------------------------------------------------------------------
    def source_of(self, layer: int) -> int:
        if self.w.sources == 1:
            return 0
        return layer

    def epoch_of(self, layer: int, step: int) -> int:
        if self.w.sources == 1 and self.w.layers > 1:
            return self.w.layers * step + layer + 1       # layers share one source: a later consumer is newer
        return step + 1

    def host_rows(self, source: int, req: int) -> np.ndarray:
        s = 0 if self.w.host_alias else source
        return self.store.host_rows(s, req)

    def reclaim(self):
        """Eq. 4 reclaim at the configured step: whole requests in ascending id until their optional
        pages cover the pages of the first `reclaim_requests` holders."""
        w = self.w
        held = np.array([int((ids >= 0).sum()) for ids in self.page_ids], np.int64)
        holders = np.nonzero(held > 0)[0][:w.reclaim_requests]
        deficit = int(held[holders].sum())
        q = hsk.reclaim_plan(held, deficit)
        assert q == oracle.reclaim_plan(held, deficit)
        dropped = []
        for r in range(q):
            if held[r] > 0:
                drop = np.full_like(self.page_ids[r], -1)
                self.store.residency_set(0, r, drop)
                assert self.ora[0].residency_set(r, drop) == 0
                self.page_ids[r] = drop
                dropped.append(r)
        log(f"[harness] reclaim: deficit={deficit} q={q} dropped={len(dropped)} requests")
        return q, dropped

    # ------------------------------------------------------------------------------------------------
    def resolve(self, layer: int, step: int, check: bool = True, meta_reqs=None, fused: bool = False,
                overlap: bool = False, same_stream: bool = False):
        """One resolve call (fused: hsk_resolve_attend; overlap: hsk_resolve_fetch_attend on a deferred store,
        with the fetch on the side stream unless same_stream; the attention output is kept as res["out"])."""
        w = self.w
        src = self.source_of(layer)
        e = self.epoch_of(layer, step)
        sel = self.sel[0 if w.shared_selection else layer][step]
        d_sel = torch.from_numpy(sel).cuda()
        d_locs = torch.full_like(d_sel, -7)
        d_stats = hsk.stats_tensor(self.U)
        out = None
        if fused:
            q, ad, out, scratch = self._attn_inputs(layer, step)
            self.store.resolve_attend(src, e, d_sel, d_locs, ad, q, out, scratch, stats=d_stats)
        elif overlap:
            q, ad, out, scratch = self._attn_inputs(layer, step)
            main = torch.cuda.current_stream()
            self.store.resolve_fetch_attend(src, e, d_sel, d_locs, ad, q, out, scratch, stats=d_stats, stream=main,
                                            copy_stream=main if same_stream else self.copy_stream)
        else:
            self.store.resolve_step(src, e, d_sel, d_locs, d_stats)
            if self.deferred:
                main = torch.cuda.current_stream()
                planned = torch.cuda.Event()
                planned.record(main)
                self.copy_stream.wait_event(planned)
                self.store.fetch_plan(src, stream=self.copy_stream)
                fetched = torch.cuda.Event()
                fetched.record(self.copy_stream)
                main.wait_event(fetched)
        locs = d_locs.cpu().numpy()
        stats = hsk.stats_to_numpy(d_stats)
        st = self.store.sync_status()
        res = {"sel": sel, "d_sel": d_sel, "d_locs": d_locs, "locs": locs, "stats": stats, "src": src, "status": st,
               "out": out}
        self.host_fetch.append((step, layer, int(stats["n_miss"].sum()), int(stats["n_sel"].sum())))
        if not check:
            return res
        o = self.ora[src].resolve(e, sel)
        assert o["rc"] == 0
        bad = np.argwhere(locs != o["locs"])
        assert bad.size == 0, f"locs differ at {bad[:5].tolist()} gpu={locs[tuple(bad[0])]} ora={o['locs'][tuple(bad[0])]}"
        for f in oracle.STATS_DTYPE.names:
            if f == "pad":
                continue
            g = stats[f]
            assert np.array_equal(g, o["stats"][f]), f"stats.{f} differ: gpu={g[:8]} ora={o['stats'][f][:8]}"
        for r in range(self.U):
            pos, dst = self.store.read_plan(src, r)
            opos, odst = o["plan"][r]
            assert np.array_equal(pos, opos) and np.array_equal(dst, odst), f"plan differs for request {r}"
        if meta_reqs is None:
            meta_reqs = range(self.U) if (step % self.check_meta_every == 0) else []
        for r in meta_reqs:
            g = self.store.snapshot(src, r)
            a = self.ora[src].snapshot(r)
            assert np.array_equal(g["key"], a["key"]), f"key differs r={r}"
            assert np.array_equal(g["rec"], a["rec"]), f"rec differs r={r}"
            assert np.array_equal(g["order"], a["order"]), f"order differs r={r}"
            assert np.array_equal(g["pt"], a["pt"]), f"page table differs r={r}"
            if self.page_rows:
                assert np.array_equal(g["opt"], a["opt"]), f"optional map differs r={r}"
        res["oracle"] = o
        return res

    def check_bytes(self, res, source: int | None = None, reqs=None):
        """Eq. 12: pool rows at the emitted locations hold the selected host rows, byte for byte."""
        src = res["src"] if source is None else source
        pool = self.store.pool_rows(src)
        sel = res["sel"]
        reqs = range(self.U) if reqs is None else reqs
        for r in reqs:
            got = pool.index_select(0, res["d_locs"][r].reshape(-1).long()).cpu().numpy()
            want = self.host_rows(src, r)[sel[r].reshape(-1)]
            assert np.array_equal(got, want), f"pool bytes differ from host rows for request {r}"

    # ------------------------------------------------------------------------------------------------
    def _attn_inputs(self, layer: int, step: int):
        w = self.w
        q_np = synth.queries(w, layer, step)
        q = torch.from_numpy(q_np.view(np.int16)).cuda()
        if w.kind == "mla":
            ad = hsk.mla_desc(requests=w.requests, max_queries=w.queries, heads=w.heads, dk=w.dk, dv=w.dv,
                              top_k=w.top_k, row_elems=w.row_elems, scale=w.scale)
            out = torch.zeros((w.requests, w.queries, w.heads, w.dv), dtype=torch.int16, device="cuda")
        else:
            ad = hsk.gqa_desc(requests=w.requests, heads=w.heads, kv_heads=w.kv_heads, dh=w.dk, top_k=w.top_k,
                              page_tokens=w.page_tokens, scale=w.scale)
            out = torch.zeros((w.requests, w.heads, w.dk), dtype=torch.int16, device="cuda")
        scratch = torch.empty(hsk.attn_scratch_bytes(ad), dtype=torch.uint8, device="cuda")
        return q, ad, out, scratch

    def run_attention(self, layer: int, step: int, res, source: int | None = None):
        """hsk_sparse_decode_attn on the resolved locations; returns the bf16 output (int16 view)."""
        src = res["src"] if source is None else source
        q, ad, out, scratch = self._attn_inputs(layer, step)
        hsk.sparse_decode_attn(ad, q, self.store.pool_base(src), res["d_locs"], None, out, scratch, scratch.numel())
        torch.cuda.synchronize()
        return out

    def attention(self, layer: int, step: int, res, samples=None, source: int | None = None):
        """Run the HIP attention on the resolved locations and compare sampled queries with the fp64
        oracle computed from host rows at the selected positions.  Returns (max_abs, max_rel)."""
        out = self.run_attention(layer, step, res, source)
        return self.check_attention(layer, step, res, out, samples, source)

    def check_attention(self, layer: int, step: int, res, out, samples=None, source: int | None = None):
        """Compare a bf16 attention output with the fp64 oracle on sampled queries (MLA: (request, query)
        pairs; GQA: units).  Returns (max_abs, max_rel)."""
        w = self.w
        src = res["src"] if source is None else source
        q_np = synth.queries(w, layer, step)
        got = synth.bf16_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
        sel = res["sel"]
        host_src = 0 if w.host_alias else src
        worst_abs, worst_rel = 0.0, 0.0
        if w.kind == "mla":
            pairs = [(r, j) for r in range(w.requests) for j in range(w.queries)] if samples is None else samples
            for r, j in pairs:
                rows = synth.kv_rows_at(w, host_src, r, sel[r, j])
                ref = oracle.mla_attention(q_np[r, j], rows, w.dk, w.dv, w.scale)
                g = got[r, j]
                err = np.abs(g - ref)
                assert np.all(err <= ATOL + RTOL * np.abs(ref)), \
                    f"attention r={r} j={j}: max abs err {err.max():.3e}"
                worst_abs = max(worst_abs, float(err.max()))
                worst_rel = max(worst_rel, float((err / np.maximum(np.abs(ref), 1e-3)).max()))
        else:
            gsz = w.heads // w.kv_heads
            units = range(self.U) if samples is None else samples
            for u in units:
                r, g_ = divmod(u, w.kv_heads)
                pages = synth.kv_rows_at(w, host_src, u, sel[u, 0])
                ref = oracle.gqa_attention(q_np[r, g_ * gsz:(g_ + 1) * gsz], pages, w.page_tokens, w.dk, w.scale)
                g = got[r, g_ * gsz:(g_ + 1) * gsz]
                err = np.abs(g - ref)
                assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"gqa attention unit={u}: max abs err {err.max():.3e}"
                worst_abs = max(worst_abs, float(err.max()))
                worst_rel = max(worst_rel, float((err / np.maximum(np.abs(ref), 1e-3)).max()))
        return worst_abs, worst_rel

    def close(self):
        self.store.close()
