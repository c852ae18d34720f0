"""The attention call inside a HIP graph: hsk_sparse_decode_attn_noalloc (split-k scratch in the library's static
buffer, so a captured call allocates nothing) and hsk_sparse_decode_attn with a caller buffer allocated before
capture.  The graph holds only kernels (no memset nodes).  It is replayed several times, with the program's own
eager work (other attention calls through the same static buffer, input updates) and synchronisations between
the replays, and every replay is checked against an eager call on the same inputs: same kernels and partitions,
so bit for bit.  The first replay's output is also checked against the fp64 oracle."""
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


def _inputs(R, H, k, n_rows, seed):
    g = torch.Generator().manual_seed(seed)
    rows = torch.randn((n_rows, 576), generator=g).to(torch.bfloat16)
    q = torch.randn((R, 1, H, 576), generator=g).to(torch.bfloat16)
    locs = torch.randint(0, n_rows, (R, 1, k), generator=g, dtype=torch.int32)
    return rows, q, locs


@pytest.mark.parametrize("noalloc", [True, False])
def test_attention_in_a_graph_replays_match_eager(noalloc):
    R, H, k, n = 16, 128, 1024, 8000
    rows, q, locs = _inputs(R, H, k, n, seed=11 + noalloc)
    pool = rows.view(torch.int16).cuda()
    d_q = q.view(torch.int16).cuda()
    d_locs = locs.cuda()
    ad = hsk.mla_desc(requests=R, max_queries=1, heads=H, dk=576, dv=512, top_k=k, row_elems=576,
                      scale=576 ** -0.5)
    nb = hsk.attn_scratch_bytes(ad)
    scratch = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.zeros((R, 1, H, 512), dtype=torch.int16, device="cuda")
    eager = torch.zeros_like(out)

    def call(o, stream=None):
        if noalloc:
            hsk.sparse_decode_attn_noalloc(ad, d_q, pool.data_ptr(), d_locs, None, o, stream=stream)
        else:
            hsk.sparse_decode_attn(ad, d_q, pool.data_ptr(), d_locs, None, o, scratch, nb, stream=stream)

    call(out)                       # eager first: the library looks up its static buffer outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call(out, stream=side)
    torch.cuda.synchronize()
    # a second, unrelated eager shape shares the static buffer between replays
    rows2, q2, locs2 = _inputs(3, 64, 300, 2000, seed=99)
    ad2 = hsk.mla_desc(requests=3, max_queries=1, heads=64, dk=576, dv=512, top_k=300, row_elems=576,
                       scale=576 ** -0.5)
    pool2, q2d, l2d = rows2.view(torch.int16).cuda(), q2.view(torch.int16).cuda(), locs2.cuda()
    nb2 = hsk.attn_scratch_bytes(ad2)
    sc2 = torch.empty(nb2, dtype=torch.uint8, device="cuda")
    other = torch.zeros((3, 1, 64, 512), dtype=torch.int16, device="cuda")
    for rep in range(4):
        if rep == 2:                # new inputs in place: the replay must read them
            d_q.copy_(torch.randn((R, 1, H, 576)).to(torch.bfloat16).view(torch.int16))
            d_locs.copy_(torch.randint(0, n, (R, 1, k), dtype=torch.int32))
        out.fill_(33)
        graph.replay()
        torch.cuda.synchronize()
        call(eager)
        if noalloc:
            hsk.sparse_decode_attn_noalloc(ad2, q2d, pool2.data_ptr(), l2d, None, other)
        else:
            hsk.sparse_decode_attn(ad2, q2d, pool2.data_ptr(), l2d, None, other, sc2, nb2)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        print(f"[graph noalloc={noalloc}] replay {rep}: identical to eager", flush=True)
        if rep == 0:
            got = synth.bf16_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
            qb = d_q.cpu().numpy().view(np.uint16)
            pr = pool.cpu().numpy().view(np.uint16)
            lc = d_locs.cpu().numpy()
            for r in (0, R - 1):
                ref = oracle.mla_attention(qb[r, 0], pr[lc[r, 0]], 576, 512, 576 ** -0.5)
                assert np.all(np.abs(got[r, 0] - ref) <= ATOL + RTOL * np.abs(ref)), r
