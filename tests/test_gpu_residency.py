"""GPU parity of scheduled residency (Adaptive DHiSparse section 3.1, Eqs. 3-4) through the C ABI.

Random scripts of admissions (resident-first from device rows, or host-first from host rows), releases,
bounded round-robin populations, publications and resolves run on the library and on the oracle's
scheduler (oracle/residency.py) side by side.  After every operation the per-page state (page id, ready,
backed) and the scheduler counters must be identical; after every resolve the locations, statistics, miss
plans, metadata and the pool bytes at every location (the selected row of the slot's current request) must
match.  Host rows of slots admitted resident-first start as a sentinel, so a resolve that fetched a row
whose host copy was never written would be caught by the byte check; after a reclaim the backed-up host
rows must hold the request's rows.  Population copies run on a second stream; the test publishes with
wait = 1 before each population so that publication points match the oracle's.
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
from oracle.residency import Residency, EWAIT, ESTATE  # noqa: E402
from hsk_harness import log  # noqa: E402

SENTINEL = 0x5A


class Pair:
    """The library store and the oracle scheduler over the same shape."""

    def __init__(self, R, S, B, T, P, pool_pages, max_ctx, k, capacity, reserve, required, per_attempt, seed,
                 optional=True, copy_stream=True):
        self.w = synth.WORKLOADS["tiny"].scaled(seed=seed)
        self.R, self.S, self.B, self.T, self.P, self.k = R, S, B, T, P, k
        self.st = hsk.KVStore(requests=R, sources=S, row_bytes=self.w.row_bytes, hot_slots=B, tail_rows=T, ctx=1,
                              max_ctx=max_ctx, page_rows=P, opt_pool_pages=pool_pages, max_queries=1, top_k=k)
        self.st.residency_init(capacity, reserve, required, per_attempt, optional)
        self.srcs = [oracle.Source(R=R, ctx=1, B=B, T=T, page_rows=P, opt_pool_pages=pool_pages,
                                   row_bytes=self.w.row_bytes, max_ctx=max_ctx) for _ in range(S)]
        self.ora = Residency(self.srcs, capacity, reserve, required, per_attempt, optional)
        self.uid = [-1] * R
        self.next_uid = 1000
        self.epoch = 0
        self.main = torch.cuda.current_stream()
        self.copy = torch.cuda.Stream() if copy_stream else self.main

    # ---- operations -------------------------------------------------------------------------------------
    def admit(self, r, n, on_device):
        uid = self.next_uid
        torch.cuda.synchronize()                        # the slot's host rows are rewritten below
        for s in range(self.S):
            self.st.host_rows(s, r)[:] = SENTINEL
        hist = None
        if on_device:
            hist = torch.from_numpy(np.stack([synth.kv_rows(self.w, s, uid, 0, n) for s in range(self.S)])
                                    .view(np.int16)).cuda()
        else:
            for s in range(self.S):
                synth.fill_kv_rows(self.st.host_ptr(s, r), self.w, s, uid, 0, n)
        want_rc, want_taken = self.ora.admit(r, n, uid, on_device)
        try:
            got = self.st.admit(r, n, hist, stream=self.main)
            rc = hsk.HSK_OK
        except hsk.HskError as e:
            rc, got = e.status, []
        assert rc == want_rc, (rc, want_rc)
        assert got == want_taken
        if rc == hsk.HSK_OK:
            self.next_uid += 1
            self.uid[r] = uid
        torch.cuda.synchronize()                        # hist may be freed
        return rc

    def release(self, r):
        assert self.ora.release(r) == oracle.OK
        self.st.release(r, stream=self.main)
        self.uid[r] = -1

    def populate(self):
        self.st.publish(wait=True, stream=self.main)
        n = self.st.populate(stream=self.main, copy_stream=self.copy)
        got = self.ora.populate()
        assert n == len(got)
        return n

    def publish(self):
        assert self.st.publish(wait=True, stream=self.main) == self.ora.publish()

    def check_state(self):
        gi, oi = self.st.residency_info(), self.ora.info()
        for key, v in oi.items():
            assert gi[key] == v, (key, gi[key], v)
        for r in range(self.R):
            ids, flags = self.st.residency_pages(r)
            oids, oflags = self.ora.page_state(r)
            assert np.array_equal(ids, oids), r
            assert np.array_equal(flags, oflags), r
        self.ora.check_invariants()

    def resolve(self, rng, check_bytes=True):
        self.epoch += 1
        R, k = self.R, self.k
        sel = np.zeros((R, 1, k), np.int32)
        nq = np.zeros(R, np.int32)
        for r in range(R):
            n = self.ora.n_import[r]
            if self.ora.admitted[r] and n >= k:
                sel[r, 0] = rng.choice(n, size=k, replace=False)
                nq[r] = 1
        d_sel = torch.from_numpy(sel).cuda()
        d_nq = torch.from_numpy(nq).cuda()
        for s in range(self.S):
            d_locs = torch.full_like(d_sel, -7)
            d_stats = hsk.stats_tensor(R)
            self.st.resolve_step(s, self.epoch, d_sel, d_locs, d_stats, nq=d_nq, stream=self.main)
            assert self.st.sync_status() == 0
            o = self.srcs[s].resolve(self.epoch, sel, nq=nq)
            assert o["rc"] == 0
            locs = d_locs.cpu().numpy()
            stats = hsk.stats_to_numpy(d_stats)
            assert np.array_equal(locs, o["locs"]), "locations differ"
            for f in oracle.STATS_DTYPE.names:
                if f != "pad":
                    assert np.array_equal(stats[f], o["stats"][f]), f
            pool = self.st.pool_rows(s)
            for r in range(R):
                if not nq[r]:
                    continue
                pos, dst = self.st.read_plan(s, r)
                assert np.array_equal(pos, o["plan"][r][0]) and np.array_equal(dst, o["plan"][r][1])
                g, a = self.st.snapshot(s, r), self.srcs[s].snapshot(r)
                for key in ("key", "rec", "order", "pt", "opt"):
                    assert np.array_equal(g[key], a[key]), (key, r)
                if check_bytes:
                    got = pool.index_select(0, d_locs[r].reshape(-1).long()).cpu().numpy()
                    want = synth.kv_rows_at(self.w, s, self.uid[r], sel[r].reshape(-1)).view(np.uint8)
                    assert np.array_equal(got, want.reshape(got.shape)), f"pool bytes, source {s} slot {r}"
        return sel, nq

    def check_backups(self):
        """Host rows of every backed complete page of an admitted request hold its rows."""
        torch.cuda.synchronize()
        for r in range(self.R):
            if not self.ora.admitted[r]:
                continue
            n = self.ora.n_import[r]
            backed = [g for g in range(n // self.P) if self.ora.backed[r][g]]
            for s in range(self.S):
                h = self.st.host_rows(s, r)
                for g in backed:
                    want = synth.kv_rows(self.w, s, self.uid[r], g * self.P, self.P).view(np.uint8)
                    assert np.array_equal(h[g * self.P:(g + 1) * self.P], want.reshape(self.P, -1)), (r, g)

    def close(self):
        torch.cuda.synchronize()
        self.st.close()


@pytest.mark.parametrize("seed,copy_stream", [(0, True), (1, False), (2, True)])
def test_random_scripts_match_the_oracle(seed, copy_stream):
    rng = np.random.default_rng(seed)
    p = Pair(R=6, S=2, B=48, T=8, P=16, pool_pages=40, max_ctx=720, k=24, capacity=44, reserve=3, required=5,
             per_attempt=3, seed=700 + seed, copy_stream=copy_stream)
    counts = {"admit": 0, "wait": 0, "release": 0, "populate": 0, "resolve": 0}
    for step in range(90):
        op = rng.choice(["admit", "release", "populate", "publish", "resolve"], p=[0.3, 0.12, 0.25, 0.08, 0.25])
        if op == "admit":
            free = [r for r in range(p.R) if not p.ora.admitted[r]]
            if not free:
                continue
            rc = p.admit(int(rng.choice(free)), int(rng.integers(1, 721)), bool(rng.integers(0, 2)))
            counts["wait" if rc == EWAIT else "admit"] += 1
        elif op == "release":
            adm = [r for r in range(p.R) if p.ora.admitted[r]]
            if adm:
                p.release(int(rng.choice(adm)))
                counts["release"] += 1
        elif op == "populate":
            p.populate()
            counts["populate"] += 1
        elif op == "publish":
            p.publish()
        else:
            p.resolve(rng)
            counts["resolve"] += 1
        p.check_state()
    p.check_backups()
    log(f"[residency seed={seed}] {counts}")
    assert counts["admit"] > 5 and counts["resolve"] > 5
    p.close()


def test_load_step_coverage_matches_the_oracle():
    """C4 -> C12 -> C4 with resident-first admissions (the small case of the oracle's load-step test):
    coverage and the host-fetched share of every step equal the oracle's, and so does every resolve."""
    rng = np.random.default_rng(5)
    R, P = 12, 16
    p = Pair(R=R, S=1, B=64, T=8, P=P, pool_pages=200, max_ctx=256, k=32, capacity=12 * 6 + 2, reserve=2,
             required=6, per_attempt=2, seed=77)
    cov, host_share = [], []
    for phase, conc in enumerate((4, 12, 4)):
        if phase == 2:
            for r in range(4, R):
                p.release(r)
        for r in range(conc):
            if not p.ora.admitted[r]:
                assert p.admit(r, 256, on_device=True) == hsk.HSK_OK
        for _ in range(30):
            p.populate()
            p.check_state()
            p.resolve(rng)
            i = p.st.residency_info()
            cov.append(i["ready_pages"] / i["eligible_pages"])
    p.check_backups()
    log(f"[load step] coverage {['%.2f' % c for c in cov[::3]]}")
    # C4: (74 - 2 - 4*6) / (4*16) = 75% of the history fits; C12: required allocations take everything
    assert cov[0] == 0.75 and min(cov[30:60]) == 0.0 and cov[-1] == 0.75
    p.close()


def test_wait_and_state_errors_change_nothing():
    p = Pair(R=3, S=1, B=16, T=4, P=8, pool_pages=8, max_ctx=64, k=8, capacity=9, reserve=2, required=4,
             per_attempt=4, seed=9)
    assert p.admit(0, 64, on_device=True) == hsk.HSK_OK          # 9-2-4 = 3 pages kept
    p.check_state()
    before = (p.st.residency_info(), [p.st.residency_pages(r) for r in range(3)])
    assert p.admit(1, 64, on_device=True) == EWAIT               # needs 4, 3 held
    assert p.admit(1, 16, on_device=False) == EWAIT
    after = (p.st.residency_info(), [p.st.residency_pages(r) for r in range(3)])
    assert before[0] == after[0]
    assert all(np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) for a, b in zip(before[1], after[1]))
    for call, status in ((lambda: p.st.admit(0, 8), hsk.HSK_ESTATE), (lambda: p.st.release(1), hsk.HSK_ESTATE),
                         (lambda: p.st.admit(1, 65), hsk.HSK_EINVAL), (lambda: p.st.admit(1, 0), hsk.HSK_EINVAL),
                         (lambda: p.st.residency_set(0, 0, [0]), hsk.HSK_ESTATE),
                         (lambda: p.st.commit_prefill(), hsk.HSK_ESTATE),
                         (lambda: p.st.residency_init(10, 0, 1, 1), hsk.HSK_ESTATE)):
        with pytest.raises(hsk.HskError) as e:
            call()
        assert e.value.status == status
    p.resolve(np.random.default_rng(1))                          # the store still works
    p.close()


def test_appends_skip_free_slots_and_admitted_rows_resolve():
    """Appends grow admitted slots only: a free slot keeps context -1 and its host rows are not written."""
    R, S, B, T, P, k = 4, 1, 32, 8, 16, 12
    p = Pair(R=R, S=S, B=B, T=T, P=P, pool_pages=16, max_ctx=300, k=k, capacity=100, reserve=0, required=2,
             per_attempt=4, seed=31)
    torch.cuda.synchronize()
    for r in range(R):
        p.st.host_rows(0, r)[:] = SENTINEL
    assert p.admit(1, 200, on_device=True) == hsk.HSK_OK
    assert p.admit(3, 150, on_device=False) == hsk.HSK_OK
    rows = torch.full((R, 2, p.w.row_elems), 7, dtype=torch.int16, device="cuda")
    for _ in range(3):
        p.st.append_rows(0, rows, 2, stream=p.main)
    torch.cuda.synchronize()
    assert [p.st.context_rows(0, r) for r in range(R)] == [-1, 206, -1, 156]
    for r in (0, 2):
        assert np.all(p.st.host_rows(0, r) == SENTINEL), f"free slot {r} was written"
    for r, n in ((1, 200), (3, 150)):
        h = p.st.host_rows(0, r)[n:n + 6]
        assert np.all(h.view(np.int16) == 7), f"appended rows of slot {r} not written through"
    p.release(1)
    assert p.st.context_rows(0, 1) == -1
    assert p.admit(1, 64, on_device=False) == hsk.HSK_OK
    assert p.st.context_rows(0, 1) == 64
    p.close()
