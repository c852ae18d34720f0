"""Load-adaptive residency in the oracle (Adaptive DHiSparse section 3.1, Eqs. 3-4), pinned to a hand-worked
round-robin example, a closed form for the round robin with ample capacity, an independent brute-force
reclaim choice, the Eq. 3 capacity bound and the guarantee that every history row is ready on the device
or backed on host -- under random admit / release / populate / resolve scripts."""
import itertools

import numpy as np
import pytest

import oracle
from oracle.residency import Residency, EWAIT, ESTATE, FLAG_READY, FLAG_BACKED


def _make(R=4, P=4, pool_pages=64, B=8, T=2, max_ctx=64, sources=1, **kw):
    srcs = [oracle.Source(R=R, ctx=np.full(R, P), B=B, T=T, page_rows=P, opt_pool_pages=pool_pages, row_bytes=16,
                          max_ctx=max_ctx) for _ in range(sources)]
    kw.setdefault("capacity_pages", 10_000)
    kw.setdefault("reserve_pages", 0)
    kw.setdefault("required_pages", 1)
    kw.setdefault("pages_per_attempt", 4)
    return Residency(srcs, **kw), srcs


def test_round_robin_worked_example():
    """3 requests with 4 complete pages each (P = 4, 16-18 rows), 4 pages per attempt, ample capacity:
    attempt 1 reserves r0 g0, r1 g0, r2 g0, r0 g1 into ids 0-3; attempt 2 continues at r1."""
    res, _ = _make(R=3, pages_per_attempt=4)
    for r, n in enumerate((16, 17, 18)):
        assert res.admit(r, n, uid=10 + r, on_device=False) == (oracle.OK, [])
    assert res.populate() == [(0, 0, 0), (1, 0, 1), (2, 0, 2), (0, 1, 3)]
    info = res.info()
    assert info["pending_pages"] == 4 and info["ready_pages"] == 0
    assert res.populate() == [(1, 1, 4), (2, 1, 5), (0, 2, 6), (1, 2, 7)]
    assert res.info()["ready_pages"] == 4 and res.info()["pending_pages"] == 4
    ids, flags = res.page_state(0)
    assert ids.tolist() == [0, 3, 6, -1]
    assert flags.tolist() == [FLAG_READY | FLAG_BACKED] * 2 + [FLAG_BACKED] * 2


@pytest.mark.parametrize("n_req,L,attempts", [(3, 4, 5), (5, 3, 7), (7, 16, 3), (2, 1, 9)])
def test_round_robin_closed_form(n_req, L, attempts):
    """Ample capacity, equal page counts, cursor from slot 0: the i-th page reserved overall goes to
    request i mod n, page i div n, id i."""
    pages = 8
    res, _ = _make(R=n_req, pages_per_attempt=L, max_ctx=pages * 4)
    for r in range(n_req):
        res.admit(r, pages * 4, uid=r, on_device=False)
    got = list(itertools.chain.from_iterable(res.populate() for _ in range(attempts)))
    want = [(i % n_req, i // n_req, i) for i in range(min(attempts * L, n_req * pages))]
    assert got == want


def _brute_q(held, deficit):
    """Eq. 4 by enumeration: the smallest prefix length whose pages cover the deficit, or -1."""
    for q in range(len(held) + 1):
        if sum(held[:q]) >= deficit:
            return q
    return -1


def test_admission_reclaim_and_wait():
    """Capacity 40, 4 pages per request required, resident-first admissions: the first requests keep their
    pages; an admission that needs more reclaims whole requests oldest-first (Eq. 4), backing up their
    device-only pages before retiring them; when nothing can cover the deficit it waits and nothing changes."""
    res, srcs = _make(R=6, P=4, pool_pages=64, max_ctx=40, capacity_pages=40, reserve_pages=2, required_pages=4)
    assert res.admit(0, 40, uid=100, on_device=True) == (oracle.OK, [])     # 10 pages retained
    assert res.admit(1, 40, uid=101, on_device=True) == (oracle.OK, [])     # 40-2-8-10 = 20 -> 10 retained
    i = res.info()
    assert i["optional_pages"] == 20 and i["unbacked_pages"] == 20 and i["ready_pages"] == 20
    assert i["free_pages"] == 40 - 2 - 8 - 20 == 10
    assert res.admit(2, 20, uid=102, on_device=True) == (oracle.OK, [])     # 10-4 = 6 free -> 5 pages of 5
    assert res.info()["free_pages"] == 1
    # slot 3 needs 4 more pages: deficit 3 -> reclaim request 0 (oldest, 10 pages)
    rc, taken = res.admit(3, 8, uid=103, on_device=True)
    assert rc == oracle.OK and taken == [0]
    ids, flags = res.page_state(0)
    assert np.all(ids == -1) and np.all(flags == FLAG_BACKED)                # backed up, then retired
    assert res.info()["free_pages"] == 1 + 10 - 4 - 2                        # slot 3 kept 2 pages
    res.check_invariants()
    res2, _ = _make(R=2, P=4, capacity_pages=9, reserve_pages=2, required_pages=4)
    assert res2.admit(0, 8, uid=1, on_device=True)[0] == oracle.OK         # 9-2-4 = 3 -> 2 pages retained
    before = (res2.info(), [p.tolist() for r in range(2) for p in res2.page_state(r)])
    assert res2.admit(1, 8, uid=2, on_device=True) == (EWAIT, [])          # needs 4, only 2 pages held
    assert res2.admit(1, 8, uid=2, on_device=False)[0] == EWAIT
    assert res2.admit(0, 8, uid=3, on_device=True)[0] == ESTATE             # slot in use
    assert res2.release(1) == ESTATE
    assert (res2.info(), [p.tolist() for r in range(2) for p in res2.page_state(r)]) == before
    assert before[0]["admitted"] == 1 and before[0]["optional_pages"] == 2


def test_resident_pages_resolve_directly_and_reclaimed_rows_miss_from_host():
    """Rows of retained pages resolve from the optional pool without a host read; after their request is
    reclaimed (backup, retire) the same rows miss and are fetched from their host copies."""
    res, (src,) = _make(R=2, P=4, pool_pages=16, B=8, T=2, max_ctx=32, capacity_pages=12, reserve_pages=0,
                        required_pages=4)
    assert res.admit(0, 32, uid=7, on_device=True)[0] == oracle.OK          # 12-4 = 8 -> all 8 pages
    sel = np.zeros((2, 1, 4), np.int32)
    sel[0, 0] = [1, 5, 13, 31]                                               # 31: tail (n = 32, T = 2)
    o = src.resolve(1, sel, nq=[1, 0])
    st = o["stats"][0]
    assert int(st["n_opt"]) == 3 and int(st["n_tail"]) == 1 and int(st["n_miss"]) == 0
    assert src.pool_lookup(o["locs"][0, 0]).tolist() == [(7 << 32) | p for p in (1, 5, 13, 31)]
    rc, taken = res.admit(1, 32, uid=8, on_device=True)                    # deficit 4 -> reclaim slot 0
    assert rc == oracle.OK and taken == [0]
    o = src.resolve(2, sel, nq=[1, 0])
    st = o["stats"][0]
    assert int(st["n_opt"]) == 0 and int(st["n_miss"]) == 3 and int(st["n_tail"]) == 1
    assert o["plan"][0][0].tolist() == [1, 5, 13]
    ids, flags = res.page_state(0)
    assert all(flags[p // 4] & FLAG_BACKED for p in (1, 5, 13))
    res.check_invariants()


def test_pending_pages_stay_out_of_the_map_until_published():
    res, (src,) = _make(R=1, P=4, pool_pages=8, B=8, T=2, max_ctx=32, pages_per_attempt=2)
    res.admit(0, 32, uid=3, on_device=False)
    assert res.populate() == [(0, 0, 0), (0, 1, 1)]
    sel = np.array([[[0, 4, 9, 12]]], np.int32)
    o = src.resolve(1, sel)
    assert int(o["stats"]["n_opt"][0]) == 0 and int(o["stats"]["n_miss"][0]) == 4   # pending: hot-cache path
    assert res.publish() == 2
    o = src.resolve(2, sel)
    assert int(o["stats"]["n_opt"][0]) == 2                                  # pages 0 and 1 ready now
    assert o["locs"][0, 0, :2].tolist() == [8 + 2 + 0 * 4 + 0, 8 + 2 + 1 * 4 + 0]   # R*B + R*T + id*P + p%P


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_scripts_keep_eq3_and_host_backing(seed):
    """Random admit / release / populate / publish / resolve scripts on two sources: after every operation
    Eq. 3 holds, page ids are unique, every history row is ready or backed, each admission's reclaim set is
    the brute-force Eq. 4 prefix in admission order, and no resolve ever plans a host read of a row whose
    page is device-only."""
    rng = np.random.default_rng(seed)
    R, P, B, T, k = 6, 4, 16, 2, 6
    res, srcs = _make(R=R, P=P, pool_pages=40, B=B, T=T, max_ctx=48, sources=2, capacity_pages=44,
                      reserve_pages=3, required_pages=5, pages_per_attempt=3)
    uid, epoch = 0, 0
    for _ in range(300):
        op = rng.choice(["admit", "release", "populate", "publish", "resolve"], p=[0.3, 0.15, 0.25, 0.1, 0.2])
        if op == "admit":
            free = [r for r in range(R) if not res.admitted[r]]
            if not free:
                continue
            r = int(rng.choice(free))
            n = int(rng.integers(1, 49))
            order = sorted((x for x in range(R) if res.admitted[x]), key=lambda x: res.seq[x])
            held = [sum(1 for i in res.ids[x] if i >= 0) for x in order]
            deficit = res.required_in_use() + 5 + res.optional_in_use() + 3 - 44
            q = _brute_q(held, deficit) if deficit > 0 else 0
            uid += 1
            rc, taken = res.admit(r, n, uid, on_device=bool(rng.integers(0, 2)))
            if q < 0:
                assert rc == EWAIT
            else:
                assert rc == oracle.OK and taken == order[:q]
        elif op == "release":
            adm = [r for r in range(R) if res.admitted[r]]
            if adm:
                assert res.release(int(rng.choice(adm))) == oracle.OK
        elif op == "populate":
            got = res.populate()
            assert len(got) <= 3
        elif op == "publish":
            res.publish()
        else:
            epoch += 1
            sel = np.zeros((R, 1, k), np.int32)
            nq = np.zeros(R, np.int32)
            for r in range(R):
                if res.admitted[r] and res.n_import[r] >= k:
                    sel[r, 0] = rng.choice(res.n_import[r], size=k, replace=False)
                    nq[r] = 1
            for s in srcs:
                o = s.resolve(epoch, sel, nq=nq)
                assert o["rc"] == 0
                for r in range(R):
                    for p in o["plan"][r][0]:
                        g = int(p) // P
                        if g < len(res.ids[r]):
                            assert res.backed[r][g], f"host read of device-only row {p} of slot {r}"
                    if nq[r]:
                        want = (s.snapshot(r)["opt"] >= 0).sum()
                        assert want == sum(1 for g in range(len(res.ids[r])) if res.ready[r][g])
        res.check_invariants()
        i = res.info()
        assert i["required_pages"] + i["optional_pages"] + 3 <= 44


def test_load_step_shape():
    """A small C4 -> C12 -> C4 load step with resident-first admissions: coverage starts high, falls to
    zero while required allocations fill the capacity, and recovers through bounded repopulation after the
    load falls (the shape of Adaptive DHiSparse Figure 6b)."""
    R, P = 12, 4
    res, _ = _make(R=R, P=P, pool_pages=200, B=8, T=2, max_ctx=64, capacity_pages=12 * 6 + 2,
                   reserve_pages=2, required_pages=6, pages_per_attempt=2)
    cov = []
    uid = 0
    for phase, conc in enumerate((4, 12, 4)):
        if phase == 2:
            for r in range(4, R):
                res.release(r)
        for r in range(conc):
            if not res.admitted[r]:
                uid += 1
                assert res.admit(r, 64, uid, on_device=True)[0] == oracle.OK
        for _ in range(40):
            res.populate()
            res.check_invariants()
            i = res.info()
            cov.append(i["ready_pages"] / max(1, i["eligible_pages"]))
    # C4: (74 - 2 - 4*6) / 64 = 75% of the history fits; C12: required allocations take everything
    assert cov[0] == 0.75 and min(cov[40:80]) == 0.0 and cov[-1] == 0.75
