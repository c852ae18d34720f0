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
