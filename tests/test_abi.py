"""The C-ABI library loads, exports what include/hsk.h declares, and its host-only logic is right (CPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def hsk():
    import hierarchical_sparse_kv_layer_amd as h
    return h


def test_library_exports_every_declared_symbol(hsk):
    decl = set(re.findall(r"\b(hsk_[a-z_]+)\s*\(", open(os.path.join(ROOT, "include", "hsk.h")).read()))
    assert decl == set(hsk.EXPORTS)
    lib = ctypes.CDLL(hsk.LIB_PATH)
    for name in decl:
        assert getattr(lib, name) is not None


def test_status_strings(hsk):
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert hsk.status_str(s).startswith("HSK_")
    assert hsk.status_str(-99) == "unknown hsk_status"


def _desc(hsk, w, **over):
    ctx = np.full(w.units, w.ctx, np.int64)
    kw = dict(num_requests=w.units, num_sources=w.sources, row_bytes=w.row_bytes, hot_slots=w.hot_slots,
              tail_rows=w.tail_rows, page_rows=0, opt_pool_pages=0, max_queries=w.queries, top_k=w.top_k,
              staging_rows=w.staging_rows, host_alias_sources=int(w.host_alias), max_ctx=w.ctx,
              ctx_len=ctx.ctypes.data, gather_mode=0, gather_blocks=0)
    kw.update(over)
    return hsk.Desc(**kw), ctx


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_and_pool_sizes(hsk, name):
    w = synth.WORKLOADS[name]
    opt_pages = 0
    page_rows = 0
    if w.residency_levels:
        page_rows = w.page_rows
        opt_pages = w.requests * (w.ctx // w.page_rows)
    d, ctx = _desc(hsk, w, page_rows=page_rows, opt_pool_pages=opt_pages)
    ws, pool = hsk.workspace_bytes(d)
    rows = w.units * w.hot_slots + w.units * w.tail_rows + opt_pages * page_rows + w.units * w.staging_rows
    assert pool == rows * w.sources * w.row_bytes
    # metadata: key, rec (4 B), order (2 B) per slot, page table (4 B) per row, maps, plans; one fill code
    # (4 B) per selection for the fused resolve + attend when requests carry one query
    per_src = w.units * w.hot_slots * 10 + w.units * w.ctx * 4 + 2 * 4 * w.units * w.queries * w.top_k
    fill = 4 * w.units * w.top_k if w.queries == 1 else 0
    lo = per_src * w.sources + fill
    assert lo <= ws <= lo + w.units * (w.ctx // 64 + 64) * 4 * w.sources + (1 << 20)


def test_invalid_descriptions_rejected(hsk):
    w = synth.WORKLOADS["tiny"]
    for over in (dict(row_bytes=1000), dict(hot_slots=0), dict(hot_slots=hsk.MAX_HOT_SLOTS + 1),
                 dict(tail_rows=-1), dict(max_queries=0), dict(top_k=0), dict(page_rows=0, opt_pool_pages=5),
                 dict(max_queries=64, top_k=2048), dict(gather_mode=7), dict(max_ctx=100)):
        d, ctx = _desc(hsk, w, **over)
        with pytest.raises(hsk.HskError) as e:
            hsk.workspace_bytes(d)
        assert e.value.status == hsk.HSK_EINVAL


def test_reclaim_plan_matches_oracle(hsk):
    rng = np.random.default_rng(1)
    for _ in range(300):
        a = rng.integers(0, 20, size=int(rng.integers(0, 12)))
        delta = int(rng.integers(-3, 120))
        assert hsk.reclaim_plan(a, delta) == oracle.reclaim_plan(a, delta)


def test_attention_scratch_sizes(hsk):
    d = hsk.mla_desc(requests=64, max_queries=1, heads=128, dk=576, dv=512, top_k=2048, row_elems=576, scale=0.04)
    b = hsk.attn_scratch_bytes(d)
    assert b >= 64 * 128 * 512 * 4
    bad = hsk.mla_desc(requests=64, max_queries=1, heads=100, dk=576, dv=512, top_k=2048, row_elems=576, scale=0.04)
    with pytest.raises(hsk.HskError):
        hsk.attn_scratch_bytes(bad)
    g = hsk.gqa_desc(requests=32, heads=32, kv_heads=8, dh=128, top_k=256, page_tokens=16, scale=0.088)
    assert hsk.attn_scratch_bytes(g) >= 32 * 32 * 128 * 4
    # a forced split is an upper bound whose partitions must fit: 2,049 pages in 2 would need 1,025 pages in
    # one GQA partition (1,024 at most), 8,192 rows in 3 would need 2,731 in one MLA partition (2,048 at most)
    for d in (hsk.gqa_desc(requests=3, heads=32, kv_heads=8, dh=128, top_k=2049, page_tokens=16, scale=0.088,
                           split=2),
              hsk.mla_desc(requests=2, max_queries=1, heads=128, dk=576, dv=512, top_k=8192, row_elems=576,
                           scale=0.04, split=3)):
        with pytest.raises(hsk.HskError) as e:
            hsk.attn_scratch_bytes(d)
        assert e.value.status == hsk.HSK_EINVAL
    for d in (hsk.gqa_desc(requests=3, heads=32, kv_heads=8, dh=128, top_k=2049, page_tokens=16, scale=0.088,
                           split=3),
              hsk.mla_desc(requests=2, max_queries=1, heads=128, dk=576, dv=512, top_k=8192, row_elems=576,
                           scale=0.04, split=4)):
        assert hsk.attn_scratch_bytes(d) > 0


def test_attention_rejects_non_positive_or_non_finite_scale(hsk):
    """The kernels take the maximum of the raw scores and scale it afterwards, which needs scale > 0."""
    for sc in (0.0, -0.04, float("nan"), float("inf")):
        d = hsk.mla_desc(requests=2, max_queries=1, heads=128, dk=576, dv=512, top_k=64, row_elems=576, scale=sc)
        with pytest.raises(hsk.HskError) as e:
            hsk.attn_scratch_bytes(d)
        assert e.value.status == hsk.HSK_EINVAL
        g = hsk.gqa_desc(requests=2, heads=32, kv_heads=8, dh=128, top_k=16, page_tokens=16, scale=sc)
        with pytest.raises(hsk.HskError):
            hsk.attn_scratch_bytes(g)


def test_stream_helpers_reject_null(hsk):
    """hsk_stream_create needs somewhere to put the stream; hsk_stream_destroy needs a stream (no device call)."""
    assert hsk._lib.hsk_stream_create(None) == hsk.HSK_EINVAL
    assert hsk._lib.hsk_stream_destroy(None) == hsk.HSK_EINVAL
