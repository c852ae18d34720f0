"""Pins for the oracle's attention, rounding, reclaim, sizing and location layout (CPU only)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(x):
    """float -> bf16 bit patterns through torch (library rounding, RNE)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(u16):
    return synth.bf16_to_f32(u16).astype(np.float64)


# ---------------------------------------------------------------------------------------------- attention
@pytest.mark.parametrize("H,k,dk,dv", [(4, 7, 16, 8), (16, 64, 576, 512), (3, 1, 32, 32)])
def test_mla_attention_matches_library_softmax(H, k, dk, dv):
    """Adaptive DHiSparse Eq. 1: attention over the selected rows; cross-checked against torch's float64
    scaled_dot_product_attention (a library routine)."""
    rng = np.random.default_rng(H * 100 + k)
    q = _bf16(rng.standard_normal((H, dk)))
    rows = _bf16(rng.standard_normal((k, dk)))
    scale = 1 / math.sqrt(dk)
    got = oracle.mla_attention(q, rows, dk, dv, scale)
    Q = torch.from_numpy(_f(q))[None, :, None, :]          # [1, H, 1, dk]
    K = torch.from_numpy(_f(rows))[None, None].expand(1, H, k, dk)
    V = torch.from_numpy(_f(rows)[:, :dv])[None, None].expand(1, H, k, dv)
    # dk != dv: compute scores with SDPA's math on the key part, then the value part explicitly
    if dk == dv:
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, :, 0].numpy()
    else:
        w = torch.softmax((Q @ K.transpose(-1, -2)) * scale, dim=-1)
        ref = (w @ V)[0, :, 0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_mla_attention_special_cases():
    rng = np.random.default_rng(3)
    H, dk, dv = 5, 64, 48
    q = _bf16(rng.standard_normal((H, dk)))
    row = _bf16(rng.standard_normal((1, dk)))
    # one selected row -> its value part
    out = oracle.mla_attention(q, row, dk, dv, 0.125)
    np.testing.assert_array_equal(out, np.broadcast_to(_f(row)[0, :dv], (H, dv)))
    # identical rows -> that row's value part
    out = oracle.mla_attention(q, np.repeat(row, 9, axis=0), dk, dv, 0.125)
    np.testing.assert_allclose(out, np.broadcast_to(_f(row)[0, :dv], (H, dv)), rtol=1e-15, atol=1e-15)
    # q = 0 -> mean of the value parts
    rows = _bf16(rng.standard_normal((11, dk)))
    out = oracle.mla_attention(np.zeros((H, dk), np.uint16), rows, dk, dv, 0.125)
    np.testing.assert_allclose(out, np.broadcast_to(_f(rows)[:, :dv].mean(0), (H, dv)), rtol=1e-13, atol=1e-14)
    # the order of the selected list does not change the result
    perm = rng.permutation(11)
    a = oracle.mla_attention(q, rows, dk, dv, 0.3)
    b = oracle.mla_attention(q, rows[perm], dk, dv, 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_gqa_attention_matches_library_softmax():
    rng = np.random.default_rng(4)
    Hg, dh, kp, pt = 4, 128, 5, 16
    q = _bf16(rng.standard_normal((Hg, dh)))
    pages = _bf16(rng.standard_normal((kp, pt * 2 * dh)))
    scale = 1 / math.sqrt(dh)
    got = oracle.gqa_attention(q, pages, pt, dh, scale)
    tok = _f(pages).reshape(kp * pt, 2 * dh)
    K = torch.from_numpy(tok[:, :dh])[None, None].expand(1, Hg, kp * pt, dh)
    V = torch.from_numpy(tok[:, dh:])[None, None].expand(1, Hg, kp * pt, dh)
    Q = torch.from_numpy(_f(q))[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, :, 0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_resolved_equals_resident_tiny():
    """Attention over the pool rows the oracle resolved equals attention over the host rows at the same
    selections (spec invariant; Adaptive DHiSparse Eq. 12): the pool model names the host row of
    each location, so both gathers are the same bytes."""
    w = synth.WORKLOADS["tiny"]
    sel_all = synth.selection_stream(w, 0, steps=3)
    src = oracle.Source(R=w.requests, ctx=w.ctx, B=w.hot_slots, T=w.tail_rows, row_bytes=w.row_bytes)
    src.commit_prefill()
    for t in range(3):
        out = src.resolve(t + 1, sel_all[t])
        q = synth.queries(w, 0, t)
        tags = src.pool_lookup(out["locs"])
        for r in range(w.requests):
            pos_from_pool = (tags[r, 0] & 0xFFFFFFFF).astype(np.int32)
            assert np.all((tags[r, 0] >> 32) == r)
            a = oracle.mla_attention(q[r, 0], synth.kv_rows_at(w, 0, r, pos_from_pool), w.dk, w.dv, w.scale)
            b = oracle.mla_attention(q[r, 0], synth.kv_rows_at(w, 0, r, sel_all[t, r, 0]), w.dk, w.dv, w.scale)
            assert np.array_equal(a, b)


# ---------------------------------------------------------------------------------------------- rounding
def test_bf16_rounding_matches_library():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-39, [0.0, -0.0, 1.0, -2.5]])
    x32 = x.astype(np.float32).astype(np.float64)   # float32-exact values: no double rounding in the library
    np.testing.assert_array_equal(oracle.bf16_from_f64(x32), _bf16(x32))


def test_bf16_rounding_ties_and_double_rounding():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80)
    assert oracle.bf16_from_f64([1.0 + 2 ** -8])[0] == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6 (0x3F82)
    assert oracle.bf16_from_f64([1.0 + 3 * 2 ** -8])[0] == 0x3F82
    # just above the tie rounds up; rounding through float32 first would lose the excess and tie to even
    assert oracle.bf16_from_f64([1.0 + 2 ** -8 + 2 ** -40])[0] == 0x3F81
    assert oracle.bf16_from_f64([-(1.0 + 2 ** -8 + 2 ** -40)])[0] == 0xBF81


# ---------------------------------------------------------------------------------------------- reclaim
def test_reclaim_eq4_against_brute_force():
    """Adaptive DHiSparse Eq. 4: q = min{q' : a_1 + ... + a_q' >= Delta}; -1 when nothing covers it."""
    rng = np.random.default_rng(6)
    for _ in range(500):
        n = int(rng.integers(0, 9))
        a = rng.integers(0, 10, size=n)
        delta = int(rng.integers(-2, 50))
        want = -1
        for q in range(0, n + 1):
            if sum(a[:q]) >= delta:
                want = q
                break
        assert oracle.reclaim_plan(a, delta) == want


# ---------------------------------------------------------------------------------------------- sizing
def test_sizing_worked_examples():
    g = _golden("sizing_worked_examples.json")
    ring = oracle.ring_rows(g["ring"]["window"], g["ring"]["page_rows"], g["ring"]["k_max"])
    assert ring == g["ring"]["ring_rows"]
    gib = 35 * ring * g["ring_memory"]["bytes_per_row"] / 2 ** 30
    assert abs(gib - g["ring_memory"]["gib"]) < 0.005
    s = g["staging"]
    sh = g["staging_shape"]
    live = oracle.staging_bytes(s["live_sources"], s["slots"], sh["k_max"], sh["k"], sh["row_bytes"]) / 2 ** 30
    full = oracle.staging_bytes(s["all_layers"], s["slots"], sh["k_max"], sh["k"], sh["row_bytes"]) / 2 ** 30
    assert abs(live - s["gib_live"]) < 0.005
    assert abs(full - s["gib_all"]) < 0.05
    assert abs(full / live - s["ratio"]) < 1e-9
    # Eq. 10: within a slot, positions alive together map to different ring rows; each slot owns its own block of rows
    for t1, t2 in itertools.combinations(range(0, 3 * ring, 97), 2):
        if abs(t1 - t2) < ring:
            assert oracle.ring_addr(3, t1, ring) != oracle.ring_addr(3, t2, ring)
    assert oracle.ring_addr(1, ring - 1, ring) < oracle.ring_addr(2, 0, ring)


# ---------------------------------------------------------------------------------------------- golden
def test_fig8a_fetched_bytes():
    """Figure 8a: 32 requests, width 8, B = 4,096: shared selections fetch one query's payload
    (37.75 MB), disjoint selections eight (302 MB)."""
    g = _golden("fig8a_fetch_bytes.json")
    R, W, k, B, d = g["requests"], g["width"], g["top_k"], g["hot_slots"], g["row_bytes"]
    n = 100_000
    rng = np.random.default_rng(7)
    shared = np.stack([np.tile(rng.choice(n, size=k, replace=False), (W, 1)) for _ in range(R)]).astype(np.int32)
    disjoint = np.stack([rng.choice(n, size=W * k, replace=False).reshape(W, k) for _ in range(R)]).astype(np.int32)
    tot = {}
    for name, sel in (("shared", shared), ("disjoint", disjoint)):
        src = oracle.Source(R=R, ctx=n, B=B, T=0, staging_rows=W * k, row_bytes=d)
        out = src.resolve(1, sel)
        assert np.all(out["stats"]["status"] == 0)
        tot[name] = int(out["stats"]["fetched_bytes"].sum())
    assert abs(tot["shared"] / 1e6 - g["one_query_payload_mb"]) < 0.005
    assert round(tot["disjoint"] / 1e6) == g["disjoint_payload_mb"]
    assert tot["disjoint"] == W * tot["shared"]


def test_fig3_one_copy_per_distinct_row():
    g = _golden("fig3_shared_rows.json")
    lists = np.array([g["lists"]], np.int32)
    src = oracle.Source(R=1, ctx=100, B=16, T=0, staging_rows=0, row_bytes=2)
    out = src.resolve(1, lists)
    st = out["stats"][0]
    assert st["n_miss"] == g["distinct_fetches"] and st["n_miss_sel"] == g["selections"]
    pos, loc = out["plan"][0]
    assert len(set(pos.tolist())) == len(pos)            # each distinct row copied once
    locs = out["locs"][0]
    for p, times in g["selected_times"].items():
        where = locs[lists[0] == int(p)]
        assert where.size == times and len(set(where.tolist())) == 1   # every selecting query gets that row


def test_location_layout_hand_worked():
    """Pool row layout, worked by hand for R=2, B=4, T=2, 4-row pages, 3 optional pages, 2 staging rows
    per request:  hot rows 0..7 (request r slot s -> 4r+s), tail rows 8..11 (request r position p ->
    8 + 2r + p mod 2), optional rows 12..23 (page id g, position p -> 12 + 4g + p mod 4), staging rows
    24..27 (request r, index c -> 24 + 2r + c)."""
    src = oracle.Source(R=2, ctx=[20, 16], B=4, T=2, page_rows=4, opt_pool_pages=3, staging_rows=2, row_bytes=8)
    src.commit_prefill()
    assert src.residency_set(1, [-1, 2, -1, -1]) == 0          # request 1: page 1 (rows 4..7) -> page id 2
    sel = np.array([[[19, 18, 0, 1, 2, 3], [4, 5, 6, 7, 8, 0]],
                    [[15, 14, 5, 7, 9, 0], [13, 5, 5, 5, 5, 5]]], np.int32)
    out = src.resolve(1, sel)
    # request 0 (n=20): 19 -> tail 8 + 0 + 1 = 9; 18 -> 8; then misses in first-occurrence order
    # 0,1,2,3 -> empty slots 0,1,2,3; 4,5,6,7,8 overflow: staging holds only 2 -> whole request rejected
    assert out["stats"][0]["status"] == oracle.ESTAGE
    assert np.all(out["locs"][0] == -1)
    # request 1 (n=16): 15 -> tail 8 + 2 + 1 = 11; 14 -> 10; 5, 7 -> optional page id 2: 12 + 8 + 1 = 21, 23;
    # misses 9, 0, 13 -> slots 0, 1, 2 of request 1 -> rows 4, 5, 6
    np.testing.assert_array_equal(out["locs"][1], [[11, 10, 21, 23, 4, 5], [6, 21, 21, 21, 21, 21]])
    # second call: request 0 now fits (4 distinct misses into 4 slots); request 1 reuses its slots
    out = src.resolve(2, np.array([[[19, 18, 0, 1, 2, 3], [0, 0, 0, 0, 0, 0]],
                                   [[9, 1, 2, 3, 4, 15], [13, 13, 13, 13, 13, 13]]], np.int32))
    np.testing.assert_array_equal(out["locs"][0], [[9, 8, 0, 1, 2, 3], [0, 0, 0, 0, 0, 0]])
    # request 1: 9 hit slot 0 (row 4), 13 hit slot 2 (row 6); misses 1, 2, 3 -> slot 3 (never used), then
    # the oldest non-hit slot 1 (position 0, filled at epoch 1), then staging 0 and 1 (rows 26, 27);
    # 4 is in optional page 1 -> 12 + 8 + 0 = 20; 15 tail -> 11
    np.testing.assert_array_equal(out["locs"][1], [[4, 7, 5, 26, 20, 11], [6, 6, 6, 6, 6, 6]])
    ev_slot, ev_key = out["evictions"][1]
    assert ev_slot.tolist() == [1] and ev_key.tolist() == [0]


def test_table1_speculative_increment_is_ring_plus_staging_per_session():
    """Table 1: Adaptive DHiSparse needs 0.060 GiB more per session than Adaptive HiSparse at both 32K and
    100K context.  That is the draft ring (Eq. 9: 2,176 rows x 12,288 B per slot) plus the shared staging
    reservation (Eq. 11: four live arenas x 35 slots x 8 x 2,048 rows x 576 B), per GPU, over 35 sessions."""
    g = _golden("table1_session_memory.json")
    s = _golden("sizing_worked_examples.json")
    ring = oracle.ring_rows(s["ring"]["window"], s["ring"]["page_rows"], s["ring"]["k_max"])
    n = g["sessions_per_gpu"]
    ring_gib = n * ring * s["ring_memory"]["bytes_per_row"] / 2 ** 30
    sh = s["staging_shape"]
    stage_gib = oracle.staging_bytes(s["staging"]["live_sources"], n, sh["k_max"], sh["k"], sh["row_bytes"]) / 2 ** 30
    per_session = (ring_gib + stage_gib) / n
    for ctx in ("32K", "100K"):
        diff = g["adaptive_dhisparse_gib"][ctx] - g["adaptive_hisparse_gib"][ctx]
        assert abs(diff - g["increment_gib"]) < 5e-4
        assert abs(per_session - diff) < 1e-3, (per_session, diff)
