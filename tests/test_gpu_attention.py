"""GPU parity of the sparse decode attention kernels alone (no resolver): random pools and locations,
every head-count variant of the MLA kernel, forced and automatic split-k, ragged k, duplicate and repeated
locations, against the fp64 oracle (|gpu - ref| <= 1e-2 + 2e-2 |ref| per element)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_sparse_kv_layer_amd as hsk  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402

ATOL, RTOL = 1e-2, 2e-2


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _run_mla(R, Q, H, k, n_rows, split=0, nq=None, seed=0, row_elems=576, q_scale=1.0, make=None):
    rng = np.random.default_rng(seed)
    rows = _bf16(rng.standard_normal((n_rows, row_elems)))
    q = _bf16(q_scale * rng.standard_normal((R, Q, H, 576)))
    locs = rng.integers(0, n_rows, size=(R, Q, k)).astype(np.int32)
    if make is not None:
        rows, q, locs = make(rng, rows, q, locs)
    ad = hsk.mla_desc(requests=R, max_queries=Q, heads=H, dk=576, dv=512, top_k=k, row_elems=row_elems,
                      scale=576 ** -0.5, split=split)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    pool = torch.from_numpy(rows.view(np.int16)).cuda()
    out = torch.full((R, Q, H, 512), 77, dtype=torch.int16, device="cuda")
    d_nq = None if nq is None else torch.from_numpy(np.asarray(nq, np.int32)).cuda()
    print(f"[attn] R={R} Q={Q} H={H} k={k} split={split} rows={n_rows}", flush=True)
    hsk.sparse_decode_attn(ad, torch.from_numpy(q.view(np.int16)).cuda(), pool.data_ptr(),
                           torch.from_numpy(locs).cuda(), d_nq, out, scratch, nb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for r in range(R):
        for j in range(Q):
            if nq is not None and j >= nq[r]:
                assert np.all(got[r, j] == 77), "skipped query's output was written"
                continue
            ref = oracle.mla_attention(q[r, j], rows[locs[r, j]], 576, 512, 576 ** -0.5)
            g = synth.bf16_to_f32(got[r, j].view(np.uint16)).astype(np.float64)
            err = np.abs(g - ref)
            assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"r={r} j={j}: max abs err {err.max():.3e}"
            worst = max(worst, float(err.max()))
    return worst


@pytest.mark.parametrize("H", [16, 32, 48, 64, 128, 256])
def test_mla_head_variants(H):
    """Every wave-pair shape: 16 heads (1 pair of 16-head waves), 32/64/128 (1, 2, 4 pairs of 32), 48
    (three 16-head groups), 256 (two 128-head groups)."""
    _run_mla(R=3, Q=1, H=H, k=100, n_rows=700, seed=H)


@pytest.mark.parametrize("k,split", [(1, 0), (31, 0), (32, 1), (33, 1), (100, 3), (257, 5), (2048, 1),
                                     (2048, 0), (4096, 0)])
def test_mla_split_and_ragged_k(k, split):
    """Ragged last tiles, one row, one partition (direct bf16 output), uneven forced splits, partitions
    that end inside a tile, and k larger than one partition may hold (forced to several)."""
    _run_mla(R=2, Q=2, H=32, k=k, n_rows=5000, split=split, seed=k + split)


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("k,split", [(1, 0), (31, 0), (33, 1), (100, 3), (257, 5), (2048, 1), (2048, 0),
                                     (8192, 0), (8192, 5)])
def test_mla_32_head_waves_split_and_ragged_k(H, k, split):
    """The 32-heads-per-wave kernel (heads in 64s or 128s): ragged last tiles, one row, one partition,
    uneven forced splits, the full 2,048-row list, and 8,192 rows (more than one partition may hold: the
    automatic plan, and five partitions of 1,639 rows, so partition ends fall inside tiles and the combine
    takes its general path for more than four partitions)."""
    _run_mla(R=2, Q=1, H=H, k=k, n_rows=5000, split=split, seed=7 * k + split + H)


@pytest.mark.parametrize("H,k,split", [(128, 2048, 100), (64, 2048, 100), (32, 1000, 300), (128, 70, 64)])
def test_mla_forced_split_with_would_be_empty_partitions(H, k, split):
    """Forced splits whose ceil(k / split)-row partitions would leave the last ones empty (k = 2,048 in 100
    partitions of 21 rows: 98 hold rows; k = 70 in 64 partitions of 2 rows: 35 do): the planner makes only
    the non-empty partitions, so no partition contributes a 0/0 to the combine, for the 32-heads-per-wave
    kernel (128, 64 heads) and the 16-head-block kernel (32 heads)."""
    _run_mla(R=2, Q=1, H=H, k=k, n_rows=4000, split=split, seed=k + split + H)


@pytest.mark.parametrize("H", [64, 128])
def test_mla_score_jump_after_the_first_tile(H):
    """Scores that rise by far more than 2^64 above the first tile's maximum (one row of a late tile aligned
    with every head's query): the workgroup redoes its partition against the true maximum, and the result
    (dominated by that row) still matches the fp64 oracle; a partition without the jump is unaffected."""
    def make(rng, rows, q, locs):
        rows = _bf16(0.05 * rng.standard_normal((rows.shape[0], rows.shape[1])))
        qf = synth.bf16_to_f32(q).astype(np.float32)
        big = 3.0 * np.sign(qf[0, 0, 0])                   # aligned with head 0's query, large for all heads
        rows[17] = _bf16(np.concatenate([big, np.zeros(rows.shape[1] - 576)]))
        locs = locs.copy()
        locs[0, 0, 200] = 17                               # a late tile of the first partition of request 0
        return rows, _bf16(np.abs(qf) * np.sign(qf[0, 0, 0])), locs
    _run_mla(R=2, Q=1, H=H, k=300, n_rows=1000, split=2, seed=H, make=make)


@pytest.mark.parametrize("R,Q,H,split", [(11, 1, 128, 0), (5, 3, 128, 3), (9, 1, 64, 2), (13, 2, 16, 0)])
def test_mla_xcd_grouped_launches_with_partial_groups(R, Q, H, split):
    """Eight or more queries: the MLA workgroups and the split-k combine are grouped by XCD (query q with the
    XCD q mod 8); query counts that leave the last group of eight partial, for the 32-head-wave kernel (128
    and 64 heads) and the 16-head-block kernel."""
    _run_mla(R=R, Q=Q, H=H, k=300, n_rows=2000, split=split, seed=R * 7 + Q)


def test_mla_partial_queries_and_wide_rows():
    """Per-request query counts (outputs of skipped queries untouched), pool rows wider than the 576 key
    values (only row[0:576] is read), large score range (q scaled up)."""
    _run_mla(R=4, Q=3, H=64, k=77, n_rows=900, nq=[3, 0, 1, 2], seed=9, row_elems=640, q_scale=4.0)


def test_mla_identical_rows_and_duplicates():
    """All selected rows identical -> output = that row's values (within the bf16 tolerance: the weights
    enter the P.V product rounded to bf16); lists that repeat locations."""
    rng = np.random.default_rng(3)
    row = _bf16(rng.standard_normal(576))
    rows = np.tile(row, (50, 1))
    R, H, k = 2, 128, 64
    q = _bf16(rng.standard_normal((R, 1, H, 576)))
    locs = rng.integers(0, 50, size=(R, 1, k)).astype(np.int32)
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=H, dk=576, dv=512, top_k=k, row_elems=576,
                      scale=576 ** -0.5)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    pool = torch.from_numpy(rows.view(np.int16)).cuda()
    out = torch.empty((R, 1, H, 512), dtype=torch.int16, device="cuda")
    hsk.sparse_decode_attn(ad, torch.from_numpy(q.view(np.int16)).cuda(), pool.data_ptr(),
                           torch.from_numpy(locs).cuda(), None, out, scratch, nb)
    torch.cuda.synchronize()
    got = synth.bf16_to_f32(out.cpu().numpy().view(np.uint16))
    want = np.broadcast_to(synth.bf16_to_f32(row[:512]), got.shape)
    assert np.all(np.abs(got - want) <= ATOL + RTOL * np.abs(want))


def test_mla_rejects_unsupported_shapes():
    for kw in ({"dk": 512}, {"dv": 256}, {"heads": 24}, {"row_elems": 500}, {"top_k": 4096, "split": 1},
               {"scale": 0.0}, {"scale": -0.1}, {"scale": float("nan")}, {"scale": float("inf")}):
        args = dict(requests=1, max_queries=1, heads=16, dk=576, dv=512, top_k=8, row_elems=576, scale=0.1)
        args.update(kw)
        with pytest.raises(hsk.HskError):
            hsk.attn_scratch_bytes(hsk.mla_desc(**args))


def _run_gqa(R, H, Hkv, k, n_pages, page_tokens=16, split=0, seed=0, q_scale=1.0):
    rng = np.random.default_rng(seed)
    row_elems = page_tokens * 2 * 128
    pages = _bf16(rng.standard_normal((n_pages, row_elems)))
    q = _bf16(q_scale * rng.standard_normal((R, H, 128)))
    locs = rng.integers(0, n_pages, size=(R * Hkv, 1, k)).astype(np.int32)
    ad = hsk.gqa_desc(requests=R, heads=H, kv_heads=Hkv, dh=128, top_k=k, page_tokens=page_tokens,
                      scale=128 ** -0.5, split=split)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    pool = torch.from_numpy(pages.view(np.int16)).cuda()
    out = torch.full((R, H, 128), 77, dtype=torch.int16, device="cuda")
    print(f"[gqa] R={R} H={H} Hkv={Hkv} k={k} pages={n_pages} page_tokens={page_tokens} split={split}", flush=True)
    hsk.sparse_decode_attn(ad, torch.from_numpy(q.view(np.int16)).cuda(), pool.data_ptr(),
                           torch.from_numpy(locs).cuda(), None, out, scratch, nb)
    torch.cuda.synchronize()
    got = synth.bf16_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
    gs = H // Hkv
    for u in range(R * Hkv):
        r, g = divmod(u, Hkv)
        ref = oracle.gqa_attention(q[r, g * gs:(g + 1) * gs], pages[locs[u, 0]], page_tokens, 128, 128 ** -0.5)
        err = np.abs(got[r, g * gs:(g + 1) * gs] - ref)
        assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"unit {u}: max abs err {err.max():.3e}"


@pytest.mark.parametrize("k,split", [(1, 0), (7, 1), (7, 3), (256, 0), (256, 1), (100, 6), (100, 0), (200, 0),
                                     (10, 8), (1024, 1), (2049, 0)])
def test_gqa_pages_split_and_ragged(k, split):
    """GQA page attention: one page, ragged last tiles (k*16 not a multiple of 64 tokens), forced and
    automatic splits.  Automatic splits at R = 3, Hkv = 8 ask for 43 partitions: k = 100 (ceil 3 pages each,
    so only 34 hold pages) and k = 200 (5 pages each, 40 hold pages); the forced k = 10 in 8 (2 pages each,
    5 hold pages).  The planner makes only the non-empty partitions.  A partition at its largest, 1,024 pages
    forced into one, and 2,049 pages under the automatic plan."""
    _run_gqa(R=3, H=32, Hkv=8, k=k, n_pages=600, split=split, seed=k * 10 + split)


def test_gqa_automatic_plan_at_the_partition_limit():
    """1,024 units (128 requests x 8 KV heads) need no split for the grid, but 1,025 pages exceed what one
    partition holds: the automatic plan takes the smallest split that fits (2 partitions of 513 pages)."""
    _run_gqa(R=128, H=8, Hkv=8, k=1025, n_pages=300, seed=1025)


def test_gqa_xcd_grouped_combine_partial_group():
    """Nine requests: the split-k combine of the GQA partitions grouped by XCD with a partial last group."""
    _run_gqa(R=9, H=32, Hkv=8, k=100, n_pages=500, split=3, seed=99)


@pytest.mark.parametrize("H,Hkv,pt", [(8, 8, 16), (16, 8, 16), (32, 8, 8), (32, 8, 32), (32, 8, 1), (32, 8, 64),
                                      (32, 8, 12), (32, 8, 128)])
def test_gqa_group_sizes_and_page_sizes(H, Hkv, pt):
    """1, 2 and 4 query heads per KV head; a large score range; pages of 1 to 64 tokens (power-of-two sizes
    up to a 64-token tile: whole pages per tile), and of 12 and 128 tokens (a page split across tiles)."""
    _run_gqa(R=2, H=H, Hkv=Hkv, k=40, n_pages=300, page_tokens=pt, seed=H + pt, q_scale=3.0)
