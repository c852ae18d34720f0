"""The allocation-free attention entry point (hsk_sparse_decode_attn_noalloc), for callers that cannot
allocate: its split-k scratch is a static device buffer of the library.  Compared through the C ABI with
hsk_sparse_decode_attn (same kernels and partitions, so bit for bit) and with the fp64 oracle, on two calls in
a row, the second smaller than the first, plus a call whose scratch would exceed the buffer."""
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


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _case(R, H, k, n_rows, seed):
    rng = np.random.default_rng(seed)
    rows = _bf16(rng.standard_normal((n_rows, 576)))
    q = _bf16(rng.standard_normal((R, 1, H, 576)))
    locs = rng.integers(0, n_rows, size=(R, 1, k)).astype(np.int32)
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=H, dk=576, dv=512, top_k=k, row_elems=576,
                      scale=576 ** -0.5)
    return rows, q, locs, ad


def _both(rows, q, locs, ad):
    R, H = q.shape[0], q.shape[2]
    pool = torch.from_numpy(rows.view(np.int16)).cuda()
    d_q = torch.from_numpy(q.view(np.int16)).cuda()
    d_locs = torch.from_numpy(locs).cuda()
    nb = hsk.attn_scratch_bytes(ad)
    assert nb <= hsk.NOALLOC_SCRATCH_BYTES
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ref = torch.full((R, 1, H, 512), 77, dtype=torch.int16, device="cuda")
    got = torch.full((R, 1, H, 512), 55, dtype=torch.int16, device="cuda")
    hsk.sparse_decode_attn(ad, d_q, pool.data_ptr(), d_locs, None, ref, scratch, nb)
    hsk.sparse_decode_attn_noalloc(ad, d_q, pool.data_ptr(), d_locs, None, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_the_allocating_call_twice_then_smaller():
    # first call: 64 requests x 128 heads x 2,048 rows (several partitions per query, the 100K batch-64
    # shape); second call: a smaller one (fewer requests, ragged k) that reuses the same static buffer
    for (R, H, k, n, seed) in ((64, 128, 2048, 20000, 1), (5, 128, 300, 3000, 2)):
        rows, q, locs, ad = _case(R, H, k, n, seed)
        print(f"[noalloc] R={R} H={H} k={k} scratch={hsk.attn_scratch_bytes(ad)}", flush=True)
        ref, got = _both(rows, q, locs, ad)
        assert np.array_equal(ref, got), "no-alloc output differs from hsk_sparse_decode_attn"
        for r in (0, R // 2, R - 1):
            want = oracle.mla_attention(q[r, 0], rows[locs[r, 0]], 576, 512, 576 ** -0.5)
            g = synth.bf16_to_f32(got[r, 0].view(np.uint16)).astype(np.float64)
            err = np.abs(g - want)
            assert np.all(err <= ATOL + RTOL * np.abs(want)), f"r={r}: max abs err {err.max():.3e}"


def test_noalloc_rejects_scratch_beyond_the_static_buffer():
    ad = hsk.mla_desc(requests=64, max_queries=1, heads=128, dk=576, dv=512, top_k=2048, row_elems=576,
                      scale=576 ** -0.5, split=16)
    assert hsk.attn_scratch_bytes(ad) > hsk.NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(hsk.HskError) as e:
        hsk.sparse_decode_attn_noalloc(ad, dummy, dummy, dummy, None, dummy)
    assert e.value.status == hsk.HSK_ESCRATCH
