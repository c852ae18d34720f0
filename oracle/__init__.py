"""CPU oracle of the hierarchical sparse KV hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may import this
package.  The HIP product path never imports it and shares no code with it; both consume the same seeded
inputs from :mod:`synth`.

The arithmetic lives in ``hsk_oracle.c`` (plain C, scalar loops, fp64 attention); this module is a thin
ctypes wrapper.  See ``hsk_oracle.h`` for the passages of the pages each function follows:

* "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV Cache Management" -- section 3.2
  (hot cache, page table, LRU with hits above fills), section 3.4 (fused resolve phases), section 3.5
  (plan-then-IO prefetch);
* "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy" -- section 3.1 (optional
  residency, Eq. 4 reclaim), section 3.2 / Figure 2 (residency-aware resolution order), section 3.3
  (Eqs. 5-6 union and staging), section 3.4 (Eqs. 9-11 sizing), section 3.5 (Eq. 12 exactness).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against closed forms, an independent
brute-force LRU simulator, library softmax attention, invariants and the pages' worked examples.
"""
from __future__ import annotations

import ctypes
from typing import Optional
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, ENOMEM, ERANGE, ESTAGE, EEPOCH = 0, -1, -2, -5, -6, -7
CLS_NONE, CLS_TAIL, CLS_OPT, CLS_HIT, CLS_FILL, CLS_STAGED = 0, 1, 2, 3, 4, 5

STATS_DTYPE = np.dtype([("n_sel", np.int32), ("n_tail", np.int32), ("n_opt", np.int32), ("n_hit", np.int32),
                        ("n_hit_sel", np.int32), ("n_miss", np.int32), ("n_miss_sel", np.int32),
                        ("n_staged", np.int32), ("status", np.int32), ("pad", np.int32),
                        ("fetched_bytes", np.int64)])

_lib = None


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "hsk_oracle.c")
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", LIB_PATH + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, u32, vp, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_double
        L.ora_create.argtypes = [i32, vp, i64, i32, i32, i32, i64, i32, i32, i64]
        L.ora_create.restype = vp
        L.ora_destroy.argtypes = [vp]
        L.ora_destroy.restype = None
        L.ora_pool_rows.argtypes = [vp]
        L.ora_pool_rows.restype = i64
        L.ora_commit_prefill.argtypes = [vp]
        L.ora_commit_prefill.restype = None
        L.ora_residency_set.argtypes = [vp, i32, vp, i64]
        L.ora_residency_set.restype = i32
        L.ora_resolve.argtypes = [vp, u32, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.ora_resolve.restype = i32
        L.ora_set_threads.argtypes = [i32]
        L.ora_set_threads.restype = None
        L.ora_get_threads.argtypes = []
        L.ora_get_threads.restype = i32
        L.ora_promote.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
        L.ora_promote.restype = i32
        L.ora_snapshot.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        L.ora_snapshot.restype = None
        L.ora_pool_lookup.argtypes = [vp, vp, i64, vp]
        L.ora_pool_lookup.restype = None
        L.ora_mla_attention.argtypes = [vp, vp, i32, i32, i32, i32, i32, f64, vp]
        L.ora_mla_attention.restype = None
        L.ora_gqa_attention.argtypes = [vp, vp, i32, i32, i32, i32, f64, vp]
        L.ora_gqa_attention.restype = None
        L.ora_bf16_from_f64.argtypes = [vp, vp, i64]
        L.ora_bf16_from_f64.restype = None
        L.ora_reclaim_plan.argtypes = [vp, i32, i64]
        L.ora_reclaim_plan.restype = i32
        L.ora_admit.argtypes = [vp, i32, i64, i64]
        L.ora_admit.restype = i32
        L.ora_append.argtypes = [vp, i32]
        L.ora_append.restype = i32
        L.ora_context_rows.argtypes = [vp, i32]
        L.ora_context_rows.restype = i64
        L.ora_completed_rows.argtypes = [i64, i64, i32, vp, vp]
        L.ora_completed_rows.restype = i32
        L.ora_policy_replay.argtypes = [vp, i32, i32, i64, i64, i32, i32, ctypes.c_uint64, vp]
        L.ora_policy_replay.restype = i32
        L.ora_ring_rows.argtypes = [i64, i64, i64]
        L.ora_ring_rows.restype = i64
        L.ora_ring_addr.argtypes = [i64, i64, i64]
        L.ora_ring_addr.restype = i64
        L.ora_staging_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.ora_staging_bytes.restype = f64
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


class Source:
    """One payload source: R requests' hot caches (B slots), tails (T rows), optional-history page maps
    and staging rows, with a pool model of which host row each pool row holds."""

    def __init__(self, R, ctx, B, T, page_rows=0, opt_pool_pages=0, staging_rows=0, row_bytes=1152, max_ctx=None,
                 stg_base=-1):
        """stg_base: first staging row relative to the source's pool rows when staging is an arena shared
        with other sources (-1: right after the optional pages)."""
        self.R, self.B, self.T = int(R), int(B), int(T)
        self.ctx = np.array(np.broadcast_to(np.asarray(ctx, dtype=np.int64), (self.R,)))
        self.max_ctx = int(self.ctx.max() if max_ctx is None else max_ctx)
        self.page_rows, self.opt_pool_pages, self.staging_rows = int(page_rows), int(opt_pool_pages), int(staging_rows)
        self.row_bytes = int(row_bytes)
        self._h = lib().ora_create(self.R, _p(self.ctx), self.max_ctx, self.B, self.T, self.page_rows,
                                   self.opt_pool_pages, self.staging_rows, self.row_bytes, int(stg_base))
        if not self._h:
            raise ValueError("ora_create rejected the shape")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().ora_destroy(h)
            self._h = None

    @property
    def pool_rows(self) -> int:
        return int(lib().ora_pool_rows(self._h))

    def commit_prefill(self):
        lib().ora_commit_prefill(self._h)

    def residency_set(self, r: int, page_ids) -> int:
        ids = np.ascontiguousarray(np.asarray(page_ids, dtype=np.int32))
        return int(lib().ora_residency_set(self._h, int(r), _p(ids), ids.size))

    def append(self, count: int) -> int:
        """Every request's next `count` rows join the context through the tail (HiSparse 3.3 step 4)."""
        return int(lib().ora_append(self._h, int(count)))

    def context_rows(self, r: int) -> int:
        return int(lib().ora_context_rows(self._h, int(r)))

    def admit(self, r: int, n_rows: int, uid: int) -> int:
        """A new request (identity uid) takes slot r with n_rows of imported history (Adaptive DHiSparse
        3.1 admission); later pool rows of the slot are tagged (uid << 32) | position."""
        rc = int(lib().ora_admit(self._h, int(r), int(n_rows), int(uid)))
        if rc == OK:
            self.ctx[r] = int(n_rows)
        return rc

    def resolve(self, epoch: int, sel: np.ndarray, nq=None) -> dict:
        """sel int32 [R][Qmax][k].  Returns locs, cls, stats, plan (per request: positions and pool rows in
        miss order) and evictions (per request: slots and the positions they held, in victim order)."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        R, Q, k = sel.shape
        assert R == self.R
        nqa = None if nq is None else np.ascontiguousarray(np.asarray(nq, dtype=np.int32))
        locs = np.full((R, Q, k), -1, dtype=np.int32)
        cls = np.zeros((R, Q, k), dtype=np.uint8)
        stats = np.zeros(R, dtype=STATS_DTYPE)
        cap = Q * k
        plan_pos = np.zeros((R, cap), dtype=np.int32)
        plan_loc = np.zeros((R, cap), dtype=np.int32)
        plan_n = np.zeros(R, dtype=np.int32)
        ev_slot = np.zeros((R, self.B), dtype=np.int32)
        ev_key = np.zeros((R, self.B), dtype=np.int32)
        ev_n = np.zeros(R, dtype=np.int32)
        rc = lib().ora_resolve(self._h, int(epoch), _p(sel), Q, k, _p(nqa), _p(locs), _p(cls), _p(stats),
                               _p(plan_pos), _p(plan_loc), _p(plan_n), cap, _p(ev_slot), _p(ev_key), _p(ev_n))
        out = {"rc": int(rc), "locs": locs, "cls": cls, "stats": stats,
               "plan": [(plan_pos[r, :plan_n[r]].copy(), plan_loc[r, :plan_n[r]].copy()) for r in range(R)],
               "evictions": [(ev_slot[r, :ev_n[r]].copy(), ev_key[r, :ev_n[r]].copy()) for r in range(R)]}
        return out

    def promote(self, sel: np.ndarray, locs: np.ndarray, accepted, nq=None) -> np.ndarray:
        """Promotion copy-back after the last resolve (Adaptive DHiSparse 3.4): queries 0..accepted[r] are
        committed.  Returns the number of rows promoted per request."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        locs = np.ascontiguousarray(locs, dtype=np.int32)
        R, Q, k = sel.shape
        acc = np.ascontiguousarray(np.broadcast_to(np.asarray(accepted, np.int32), (R,)))
        nqa = None if nq is None else np.ascontiguousarray(np.asarray(nq, dtype=np.int32))
        out = np.zeros(R, np.int32)
        rc = lib().ora_promote(self._h, _p(sel), Q, k, _p(nqa), _p(locs), _p(acc), _p(out))
        if rc != OK:
            raise ValueError(f"ora_promote: {rc}")
        return out

    def snapshot(self, r: int) -> dict:
        n = self.context_rows(r)
        key = np.zeros(self.B, np.int32)
        rec = np.zeros(self.B, np.uint32)
        order = np.zeros(self.B, np.int32)
        pt = np.zeros(n, np.int32)
        opt = np.zeros(max(1, int(self.ctx[r]) // self.page_rows) if self.page_rows else 1, np.int32)
        lib().ora_snapshot(self._h, int(r), _p(key), _p(rec), _p(order), _p(pt), _p(opt))
        if not self.page_rows:
            opt = np.zeros(0, np.int32)
        return {"key": key, "rec": rec, "order": order, "pt": pt, "opt": opt}

    def pool_lookup(self, locs) -> np.ndarray:
        lo = np.ascontiguousarray(np.asarray(locs, dtype=np.int32).reshape(-1))
        out = np.zeros(lo.size, np.int64)
        lib().ora_pool_lookup(self._h, _p(lo), lo.size, _p(out))
        return out.reshape(np.shape(locs))


def set_threads(n: int) -> None:
    """Threads of the oracle resolve's loop over requests (results do not depend on it)."""
    lib().ora_set_threads(int(n))


def get_threads() -> int:
    return int(lib().ora_get_threads())


def mla_attention(q: np.ndarray, rows: np.ndarray, dk: int, dv: int, scale: float) -> np.ndarray:
    """fp64 attention of one query: q bf16 [H][dk], rows bf16 [k][row_elems] -> [H][dv] float64."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    H = q.shape[0]
    k, row_elems = rows.shape
    out = np.zeros((H, dv), np.float64)
    lib().ora_mla_attention(_p(q), _p(rows), k, H, dk, dv, row_elems, float(scale), _p(out))
    return out


def gqa_attention(q: np.ndarray, pages: np.ndarray, page_tokens: int, dh: int, scale: float) -> np.ndarray:
    """fp64 attention of one (request, KV head): q bf16 [Hg][dh], pages bf16 [kp][page_tokens * 2 * dh]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    pages = np.ascontiguousarray(pages, dtype=np.uint16)
    Hg = q.shape[0]
    kp = pages.shape[0]
    out = np.zeros((Hg, dh), np.float64)
    lib().ora_gqa_attention(_p(q), _p(pages), kp, page_tokens, Hg, dh, float(scale), _p(out))
    return out


def bf16_from_f64(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.zeros(a.shape, np.uint16)
    lib().ora_bf16_from_f64(_p(a), _p(out), a.size)
    return out


def reclaim_plan(pages_held, deficit: int) -> int:
    a = np.ascontiguousarray(np.asarray(pages_held, dtype=np.int64))
    return int(lib().ora_reclaim_plan(_p(a), a.size, int(deficit)))


def completed_rows(n_before: int, n_after: int, m: int):
    """Adaptive DHiSparse Eq. 8: (first, count) of the packed rows a round completes, or None if invalid."""
    first, count = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().ora_completed_rows(int(n_before), int(n_after), int(m), ctypes.addressof(first),
                                  ctypes.addressof(count))
    return None if rc else (first.value, count.value)


POLICIES = {"lru": 0, "fifo": 1, "random": 2, "belady": 3}


def policy_replay(sel: np.ndarray, n: int, B: int, policy: str, tail_from: Optional[int] = None,
                  seed: int = 0) -> np.ndarray:
    """HiSparse 4.3 / Figure 6: misses per step of one request's stream sel [steps][k] under a replacement
    policy ("lru", "fifo", "random", "belady") with B slots (B >= k)."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    steps, k = sel.shape
    out = np.zeros(steps, np.int32)
    rc = lib().ora_policy_replay(_p(sel), steps, k, int(n), int(n if tail_from is None else tail_from), int(B),
                                 POLICIES[policy], int(seed), _p(out))
    if rc:
        raise ValueError(f"ora_policy_replay rejected the input ({rc})")
    return out


def ring_rows(window: int, page_rows: int, k_max: int) -> int:
    return int(lib().ora_ring_rows(window, page_rows, k_max))


def ring_addr(slot: int, t: int, ring: int) -> int:
    return int(lib().ora_ring_addr(slot, t, ring))


def staging_bytes(live_sources: int, slots: int, k_max: int, k: int, row_bytes: int) -> float:
    return float(lib().ora_staging_bytes(live_sources, slots, k_max, k, row_bytes))
