"""Seeded input generators: determinism and the workload statistics they promise (CPU only)."""
import ctypes

import numpy as np

import synth


def test_rows_deterministic_and_thread_independent():
    w = synth.WORKLOADS["tiny"]
    a = np.empty((3000, w.row_elems), np.uint16)
    b = np.empty((3000, w.row_elems), np.uint16)
    synth.lib().synth_rows_bf16(ctypes.c_void_p(a.ctypes.data), w.seed, synth.DOMAIN_KV, 0, 1, 100, 3000,
                                w.row_elems, 1)
    synth.lib().synth_rows_bf16(ctypes.c_void_p(b.ctypes.data), w.seed, synth.DOMAIN_KV, 0, 1, 100, 3000,
                                w.row_elems, 7)
    assert np.array_equal(a, b)
    c = synth.kv_rows_at(w, 0, 1, np.arange(100, 3100)[::-1])
    assert np.array_equal(c[::-1], a)
    f = synth.bf16_to_f32(a).astype(np.float64)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1.0) < 0.01
    assert not np.array_equal(synth.kv_rows(w, 0, 2, 100, 10), a[:10])


def test_single_query_streams():
    w = synth.WORKLOADS["tiny"]
    s = synth.selection_stream(w, 0)
    assert s.shape == (w.steps, w.requests, 1, w.top_k)
    keep = w.keep_count(w.top_k)
    assert keep == 179
    for t in range(w.steps):
        for r in range(w.requests):
            lst = s[t, r, 0]
            assert len(set(lst.tolist())) == w.top_k
            assert lst.min() >= 0 and lst.max() < w.ctx
            if t:
                assert len(set(lst.tolist()) & set(s[t - 1, r, 0].tolist())) >= keep
    assert np.array_equal(s, synth.selection_stream(w, 0))
    part = synth.selection_stream(w, 0, units=slice(2, 4))
    assert np.array_equal(part, s[:, 2:4])


def test_zipf_stream_concentrates_on_low_positions():
    w = synth.WORKLOADS["dsa100k"].scaled(requests=4, steps=3)
    s = synth.selection_stream(w, 1)
    assert w.keep_count(w.top_k) == 1638
    lst = s[0, 0, 0]
    assert len(set(lst.tolist())) == w.top_k
    assert np.median(lst) < w.ctx / 10


def test_multi_query_streams_share_a_part():
    w = synth.WORKLOADS["verify"].scaled(requests=2, steps=3)
    s = synth.selection_stream(w, 0)
    assert s.shape == (3, 2, 16, 2048)
    n_shared = w.keep_count(w.top_k, w.shared_frac)
    assert n_shared == 1229 and w.keep_count(n_shared) == 922 and w.keep_count(w.top_k - n_shared) == 614
    for t in range(3):
        common = set(s[t, 0, 0].tolist())
        for j in range(16):
            lst = s[t, 0, j]
            assert len(set(lst.tolist())) == w.top_k
            common &= set(lst.tolist())
        assert len(common) >= n_shared


def test_residency_fractions_and_pages():
    w = synth.WORKLOADS["adaptive"]
    fr = synth.residency_fractions(w)
    assert set(np.unique(fr).tolist()) <= {0.0, 0.5, 1.0} and len(np.unique(fr)) == 3
    pages = w.ctx // w.page_rows
    assert pages == 7812
    half = synth.resident_pages(w, 3, 0.5)
    assert half.size == 3906 and len(np.unique(half)) == half.size and half.max() < pages
    assert synth.resident_pages(w, 3, 1.0).size == pages and synth.resident_pages(w, 3, 0.0).size == 0
