"""Seeded synthetic inputs for the hierarchical sparse KV hot path.

This module is shared by the HIP path's tests and benchmark and by the CPU oracle's tests.  It holds
none of the method's arithmetic: it only generates inputs (KV rows, decode queries, top-k selection
streams, residency fractions) and describes the workload shapes.

Workloads (the pages evaluate on model traces and serving runs that are not available here; these
seeded synthetic inputs stand in for them with the pages' shapes):

* ``tiny``      -- MLA-shaped decode, 4 requests, 8,192-token context, 512 hot slots, 64-row tail,
                   16 heads, top-256, 70% of each step's list kept and 30% uniform over history.
* ``dsa100k``   -- DSA/MLA-shaped decode, 64 requests, 100,000-token context, 4 layers with their own
                   payloads, 4,096 hot slots, 128-row tail, 128 heads, QK dim 576, V dim 512, top-2,048,
                   80% kept and the rest Zipf(1.1) over positions.
* ``verify``    -- speculative verification, 128 requests x 16 queries, top-2,048 per query, 60% of each
                   list shared by the request's queries, 75% kept step to step, Zipf(1.1) fresh rows.
* ``adaptive``  -- load-adaptive residency, 64 requests, 500,000-token context, 2 layers sharing one
                   source, 64-row optional pages resident at 0/50/100% per request, reclaim of 16
                   requests at step 8.
* ``loadstep``  -- load step of an MLA deployment (C16 -> C256 -> C16 over four data-parallel decode GPUs),
                   one GPU's share: 52 request slots, offered concurrency 4 -> 64 -> 4, 100,000-token
                   imported histories in 64-row pages, output lengths uniform in [60, 180] steps.
* ``quest``     -- page-level GQA decode, 32 requests x 8 KV heads, 131,072 tokens in 16-token pages,
                   top-256 pages per KV head shared by 8 layers, 512 page slots per KV head.

KV rows are bf16 ~N(0,1) from a counter-based generator (see rows.c); selections come from
select.c.  Everything is a pure function of the seeds below.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# stream domains of the row generator
DOMAIN_KV = 1
DOMAIN_QUERY = 2

_lib = None


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (plain C + OpenMP)."""
    import subprocess
    srcs = [os.path.join(_HERE, "rows.c"), os.path.join(_HERE, "select.c")]
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", LIB_PATH + ".tmp"] + srcs + ["-lm"]
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
        i32, i64, u32, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p
        L.synth_rows_bf16.argtypes = [vp, u64, u32, i64, i64, i64, i64, i32, i32]
        L.synth_rows_bf16.restype = None
        L.synth_rows_at_bf16.argtypes = [vp, u64, u32, i64, i64, vp, i64, i32, i32]
        L.synth_rows_at_bf16.restype = None
        L.synth_select_single.argtypes = [vp, u64, i64, i64, i32, i32, i32, i32, i32, vp, i32]
        L.synth_select_single.restype = i32
        L.synth_select_multi.argtypes = [vp, u64, i64, i64, i32, i32, i32, i32, i32, i32, i32, i32, vp, i32]
        L.synth_select_multi.restype = i32
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "mla" or "gqa"
    requests: int             # R: requests (MLA) -- GQA resolution units are requests x kv_heads
    layers: int
    sources: int              # distinct payload sources (layers that share one source count once)
    steps: int
    ctx: int                  # context rows per request (GQA: pages per unit)
    row_elems: int            # bf16 values per stored row (MLA 576; GQA page 16 x 256)
    hot_slots: int            # B
    tail_rows: int            # T
    heads: int
    kv_heads: int
    dk: int
    dv: int
    top_k: int                # k per query
    queries: int = 1          # W / Q per request
    keep_frac: float = 0.8    # step-to-step overlap
    fresh: str = "zipf"       # "uniform" | "zipf"
    zipf_s: float = 1.1
    shared_frac: float = 0.0  # multi-query: share of each list common to the request's queries
    staging_rows: int = 0     # per request
    page_rows: int = 64       # optional-history page size
    page_tokens: int = 1      # GQA: tokens per stored page row
    residency_levels: tuple = ()     # per-request optional-history fraction choices
    reclaim_step: int = -1
    reclaim_requests: int = 0
    host_alias: bool = False  # every source reads source 0's host payload
    shared_selection: bool = False   # one selection per step shared by all layers
    seed: int = 0

    @property
    def row_bytes(self) -> int:
        return 2 * self.row_elems

    @property
    def units(self) -> int:
        """resolution units: requests (MLA) or requests x KV heads (GQA)"""
        return self.requests * (self.kv_heads if self.kind == "gqa" else 1)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)

    def keep_count(self, total: int, frac: Optional[float] = None) -> int:
        f = self.keep_frac if frac is None else frac
        return int(math.floor(f * total + 0.5))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(name="tiny", kind="mla", requests=4, layers=1, sources=1, steps=8, ctx=8192,
                     row_elems=576, hot_slots=512, tail_rows=64, heads=16, kv_heads=1, dk=576, dv=512,
                     top_k=256, keep_frac=0.7, fresh="uniform", seed=1001),
    "dsa100k": Workload(name="dsa100k", kind="mla", requests=64, layers=4, sources=4, steps=32, ctx=100_000,
                        row_elems=576, hot_slots=4096, tail_rows=128, heads=128, kv_heads=1, dk=576, dv=512,
                        top_k=2048, keep_frac=0.8, fresh="zipf", seed=2002),
    "verify": Workload(name="verify", kind="mla", requests=128, layers=4, sources=4, steps=16, ctx=100_000,
                       row_elems=576, hot_slots=4096, tail_rows=128, heads=128, kv_heads=1, dk=576, dv=512,
                       top_k=2048, queries=16, keep_frac=0.75, fresh="zipf", shared_frac=0.6,
                       staging_rows=16 * 2048, seed=3003),
    "adaptive": Workload(name="adaptive", kind="mla", requests=64, layers=2, sources=1, steps=16, ctx=500_000,
                         row_elems=576, hot_slots=4096, tail_rows=128, heads=128, kv_heads=1, dk=576, dv=512,
                         top_k=2048, keep_frac=0.8, fresh="zipf", residency_levels=(0.0, 0.5, 1.0),
                         reclaim_step=8, reclaim_requests=16, seed=4004),
    "loadstep": Workload(name="loadstep", kind="mla", requests=52, layers=1, sources=1, steps=720, ctx=100_000,
                         row_elems=576, hot_slots=4096, tail_rows=128, heads=128, kv_heads=1, dk=576, dv=512,
                         top_k=2048, keep_frac=0.8, fresh="zipf", seed=6006),
    "quest": Workload(name="quest", kind="gqa", requests=32, layers=8, sources=8, steps=16, ctx=8192,
                      row_elems=16 * 256, hot_slots=512, tail_rows=0, heads=32, kv_heads=8, dk=128, dv=128,
                      top_k=256, keep_frac=0.8, fresh="zipf", page_tokens=16, page_rows=0, host_alias=True,
                      shared_selection=True, seed=5005),
}


@dataclasses.dataclass(frozen=True)
class LoadStep:
    """Offered-load schedule of the load-step replay: phases of (offered concurrency, steps); a closed loop
    keeps that many requests in the system (admitted or waiting) and lets it drain when the load falls."""
    phases: tuple = ((4, 240), (64, 240), (4, 240))
    out_len: tuple = (60, 180)          # decode steps of a request, uniform, inclusive
    admit_per_step: int = 2             # admissions per step (the prefill side's rate)
    required_pages: int = 112           # one request's required allocation, in 64-row pages
    reserve_pages: int = 112            # admission reserve
    pages_per_attempt: int = 32         # bound of one repopulation attempt (one per step)
    templates: int = 64                 # distinct selection streams; request i follows stream i mod templates
    seed: int = 6006

    @property
    def capacity_pages(self) -> int:
        """Capacity that fits 52 admitted requests' required allocations beside the reserve."""
        return 52 * self.required_pages + self.reserve_pages


LOADSTEP = LoadStep()


def output_lengths(ls: LoadStep, n: int) -> np.ndarray:
    """Decode steps of requests 0..n-1 (seeded, uniform in ls.out_len)."""
    g = np.random.default_rng([ls.seed, 91])
    return g.integers(ls.out_len[0], ls.out_len[1] + 1, size=n)


# ----------------------------------------------------------------------------------------------
# rows and queries
# ----------------------------------------------------------------------------------------------
def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def host_source_of(w: Workload, source: int) -> int:
    """Which source's payload stream backs `source` on the host (aliasing fallback)."""
    return 0 if w.host_alias else source


def fill_kv_rows(dst_ptr: int, w: Workload, source: int, req: int, first: int, count: int,
                 nthreads: Optional[int] = None) -> None:
    """Write rows [first, first+count) of (source, request) into raw memory at dst_ptr."""
    lib().synth_rows_bf16(ctypes.c_void_p(dst_ptr), w.seed, DOMAIN_KV, host_source_of(w, source), req,
                          first, count, w.row_elems, nthreads or default_threads())


def kv_rows(w: Workload, source: int, req: int, first: int, count: int) -> np.ndarray:
    out = np.empty((count, w.row_elems), dtype=np.uint16)
    fill_kv_rows(_ptr(out), w, source, req, first, count)
    return out


def kv_rows_at(w: Workload, source: int, req: int, positions) -> np.ndarray:
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32).reshape(-1))
    out = np.empty((pos.size, w.row_elems), dtype=np.uint16)
    lib().synth_rows_at_bf16(ctypes.c_void_p(_ptr(out)), w.seed, DOMAIN_KV, host_source_of(w, source), req,
                             ctypes.c_void_p(_ptr(pos)), pos.size, w.row_elems, default_threads())
    return out


def queries(w: Workload, layer: int, step: int) -> np.ndarray:
    """Decode queries for one layer-step.

    MLA: [R][Q][H][dk] bf16 (as uint16).  GQA: [R][Hq][dk]."""
    R = w.requests
    nq = 1 if w.kind == "gqa" else w.queries
    elems = w.heads * w.dk
    out = np.empty((R, nq, elems), dtype=np.uint16)
    # one stream per (layer, step); row r * nq + j is query j of request r
    lib().synth_rows_bf16(ctypes.c_void_p(_ptr(out)), w.seed, DOMAIN_QUERY, layer, step, 0, R * nq, elems,
                          default_threads())
    if w.kind == "gqa":
        return out.reshape(R, w.heads, w.dk)
    return out.reshape(R, nq, w.heads, w.dk)


# ----------------------------------------------------------------------------------------------
# selections
# ----------------------------------------------------------------------------------------------
_cdf_cache: dict = {}


def zipf_cdf(n: int, s: float) -> np.ndarray:
    """Cumulative Zipf(s) table over ranks 1..n (rank r -> position r-1), float64."""
    key = (n, s)
    if key not in _cdf_cache:
        p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(p)
        c /= c[-1]
        _cdf_cache[key] = c
    return _cdf_cache[key]


def selection_stream(w: Workload, layer: int, steps: Optional[int] = None, units: Optional[slice] = None,
                     ) -> np.ndarray:
    """Ordered top-k lists of one layer for all its resolution units: int32 [steps][U][Q][k].

    Stream id: (layer, unit).  With ``shared_selection`` every layer uses layer 0's stream."""
    steps = w.steps if steps is None else steps
    U = w.units
    u0, u1 = (0, U) if units is None else (units.start or 0, units.stop if units.stop is not None else U)
    nb = u1 - u0
    lay = 0 if w.shared_selection else layer
    cdf = zipf_cdf(w.ctx, w.zipf_s) if w.fresh == "zipf" else None
    cdf_ptr = ctypes.c_void_p(_ptr(cdf)) if cdf is not None else None
    k = w.top_k
    if w.queries == 1:
        out = np.empty((nb, steps, k), dtype=np.int32)
        rc = lib().synth_select_single(ctypes.c_void_p(_ptr(out)), w.seed, lay, u0, nb, steps, k, w.ctx,
                                       w.keep_count(k), cdf_ptr, default_threads())
        if rc != 0:
            raise RuntimeError(f"synth_select_single failed ({rc})")
        return np.ascontiguousarray(out.transpose(1, 0, 2)).reshape(steps, nb, 1, k)
    n_shared = w.keep_count(k, w.shared_frac)
    out = np.empty((nb, steps, w.queries, k), dtype=np.int32)
    rc = lib().synth_select_multi(ctypes.c_void_p(_ptr(out)), w.seed, lay, u0, nb, steps, w.queries, k, w.ctx,
                                  n_shared, w.keep_count(n_shared), w.keep_count(k - n_shared), cdf_ptr,
                                  default_threads())
    if rc != 0:
        raise RuntimeError(f"synth_select_multi failed ({rc})")
    return np.ascontiguousarray(out.transpose(1, 0, 2, 3))


def residency_fractions(w: Workload) -> np.ndarray:
    """Per-request optional-history fraction, seeded choice from ``residency_levels``."""
    if not w.residency_levels:
        return np.zeros(w.requests)
    g = np.random.default_rng([w.seed, 77])
    return np.asarray(w.residency_levels)[g.integers(0, len(w.residency_levels), size=w.requests)]


def resident_pages(w: Workload, req: int, frac: float) -> np.ndarray:
    """Which complete optional pages of a request are resident: a seeded subset of size
    floor(frac * pages + 0.5), returned sorted."""
    pages = w.ctx // w.page_rows
    m = int(math.floor(frac * pages + 0.5))
    g = np.random.default_rng([w.seed, 78, req])
    return np.sort(g.permutation(pages)[:m]).astype(np.int64)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
