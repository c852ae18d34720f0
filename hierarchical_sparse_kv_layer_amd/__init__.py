"""hierarchical_sparse_kv_layer_amd -- Python binding of libhsk.so (MI355X / gfx950).

Argument marshalling only: every step of the hot path runs in the HIP kernels of libhsk.so (see
include/hsk.h).  PyTorch supplies device memory (tensors) and streams; the names below mirror the C ABI:

    kv_store_init / host_rows / commit_prefill / residency_set / reclaim_plan / residency_init /
    request_admit / request_release / residency_reclaim / residency_populate / residency_publish /
    residency_query / residency_pages / resolve_step /
    replay_plan / promote_staged / pool_base / sparse_decode_attn / sparse_decode_attn_noalloc / attn_scratch_bytes /
    snapshot / read_plan /
    sync_status / kv_store_destroy

The library must be built (``__graft_entry__.build()``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhsk.so")

HSK_OK, HSK_EINVAL, HSK_ENOMEM, HSK_EHIP, HSK_ESTATE, HSK_ERANGE, HSK_ESTAGE, HSK_EEPOCH = 0, -1, -2, -3, -4, -5, -6, -7
HSK_EWAIT = -8
HSK_ESCRATCH = -9
NOALLOC_SCRATCH_BYTES = 64 << 20
PAGE_READY, PAGE_BACKED = 1, 2
GATHER_ZEROCOPY, GATHER_NO_IO, GATHER_DEFERRED = 0, 1, 2
ATTN_MLA, ATTN_GQA = 0, 1
MAX_HOT_SLOTS = 8192

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: the HIP library must be built (__graft_entry__.build()); "
                      "there is no fallback path")

_i32, _i64, _u32, _vp, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float


class Desc(ctypes.Structure):
    _fields_ = [("num_requests", _i32), ("num_sources", _i32), ("row_bytes", _i32), ("hot_slots", _i32),
                ("tail_rows", _i32), ("page_rows", _i32), ("opt_pool_pages", _i64), ("max_queries", _i32),
                ("top_k", _i32), ("staging_rows", _i32), ("host_alias_sources", _i32), ("max_ctx", _i64),
                ("ctx_len", _vp), ("gather_mode", _i32), ("gather_blocks", _i32), ("staging_arenas", _i32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("kind", _i32), ("num_requests", _i32), ("max_queries", _i32), ("heads", _i32),
                ("kv_heads", _i32), ("dk", _i32), ("dv", _i32), ("top_k", _i32), ("row_elems", _i32),
                ("page_tokens", _i32), ("split", _i32), ("scale", _f32)]


class ResidencyDesc(ctypes.Structure):
    _fields_ = [("capacity_pages", _i64), ("reserve_pages", _i64), ("required_pages", _i64),
                ("pages_per_attempt", _i32), ("optional", _i32)]


class ResidencyInfo(ctypes.Structure):
    _fields_ = [("admitted", _i32), ("next_slot", _i32), ("required_pages", _i64), ("optional_pages", _i64),
                ("ready_pages", _i64), ("pending_pages", _i64), ("unbacked_pages", _i64), ("eligible_pages", _i64),
                ("free_pages", _i64)]


STATS_DTYPE = np.dtype([("n_sel", np.int32), ("n_tail", np.int32), ("n_opt", np.int32), ("n_hit", np.int32),
                        ("n_hit_sel", np.int32), ("n_miss", np.int32), ("n_miss_sel", np.int32),
                        ("n_staged", np.int32), ("status", np.int32), ("reserved", np.int32),
                        ("fetched_bytes", np.int64)])
STATS_BYTES = STATS_DTYPE.itemsize  # 48

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.POINTER
_sig = {
    "hsk_workspace_bytes": (_i32, [_P(Desc), _P(ctypes.c_size_t), _P(ctypes.c_size_t)]),
    "hsk_kv_store_init": (_i32, [_P(Desc), _vp, _vp, _vp, _P(_vp)]),
    "hsk_host_rows": (_i32, [_vp, _i32, _i32, _P(_vp), _P(_i64)]),
    "hsk_commit_prefill": (_i32, [_vp, _vp]),
    "hsk_residency_set": (_i32, [_vp, _i32, _i32, _vp, _i64, _vp]),
    "hsk_reclaim_plan": (_i32, [_vp, _i32, _i64, _P(_i32)]),
    "hsk_residency_init": (_i32, [_vp, _P(ResidencyDesc), _vp]),
    "hsk_request_admit": (_i32, [_vp, _i32, _i64, _vp, _i64, _vp, _vp, _P(_i32)]),
    "hsk_request_release": (_i32, [_vp, _i32, _vp]),
    "hsk_residency_reclaim": (_i32, [_vp, _i64, _vp, _vp, _P(_i32)]),
    "hsk_residency_populate": (_i32, [_vp, _vp, _vp, _P(_i32)]),
    "hsk_residency_publish": (_i32, [_vp, _vp, _i32, _P(_i32)]),
    "hsk_residency_query": (_i32, [_vp, _P(ResidencyInfo)]),
    "hsk_residency_pages": (_i32, [_vp, _i32, _vp, _vp, _i64, _P(_i64)]),
    "hsk_resolve_step": (_i32, [_vp, _i32, _u32, _vp, _vp, _vp, _vp, _vp]),
    "hsk_replay_plan": (_i32, [_vp, _i32, _i32, _vp]),
    "hsk_fetch_plan": (_i32, [_vp, _i32, _vp]),
    "hsk_stream_create": (_i32, [ctypes.POINTER(_vp)]),
    "hsk_stream_destroy": (_i32, [_vp]),
    "hsk_resolve_fetch_attend": (_i32, [_vp, _i32, _u32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                        _vp, _vp]),
    "hsk_promote_staged": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "hsk_append_rows": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp]),
    "hsk_context_rows": (_i32, [_vp, _i32, _i32, _P(_i64)]),
    "hsk_completed_rows": (_i32, [_i64, _i64, _i32, _P(_i64), _P(_i64)]),
    "hsk_ring_rows": (_i32, [_i64, _i32, _i32, _P(_i64)]),
    "hsk_ring_write": (_i32, [_vp, _i64, _i32, _vp, _i32, _i32, _vp, _vp]),
    "hsk_ring_window_locs": (_i32, [_i64, _i32, _i32, _vp, _vp, _vp]),
    "hsk_pool_base": (_i32, [_vp, _i32, _P(_vp)]),
    "hsk_attn_scratch_bytes": (_i32, [_P(AttnDesc), _P(ctypes.c_size_t)]),
    "hsk_sparse_decode_attn": (_i32, [_P(AttnDesc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "hsk_sparse_decode_attn_noalloc": (_i32, [_P(AttnDesc), _vp, _vp, _vp, _vp, _vp, _vp]),
    "hsk_resolve_attend": (_i32, [_vp, _i32, _u32, _vp, _vp, _vp, _P(AttnDesc), _vp, _vp, _vp, ctypes.c_size_t,
                                  _vp]),
    "hsk_snapshot": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "hsk_read_plan": (_i32, [_vp, _i32, _i32, _vp, _vp, _i32, _P(_i32)]),
    "hsk_sync_status": (_i32, [_vp, _vp]),
    "hsk_kv_store_destroy": (None, [_vp]),
    "hsk_status_str": (ctypes.c_char_p, [_i32]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_sig)


class HskError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}" if what else status_str(status))


def status_str(s: int) -> str:
    return _lib.hsk_status_str(int(s)).decode()


def _check(rc: int, what: str) -> None:
    if rc != HSK_OK:
        raise HskError(rc, what)


def _ptr(x) -> Optional[int]:
    """Device/host address of a torch tensor, numpy array or int (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------------------------------------ C ABI
def workspace_bytes(desc: Desc):
    ws, pool = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.hsk_workspace_bytes(ctypes.byref(desc), ctypes.byref(ws), ctypes.byref(pool)), "hsk_workspace_bytes")
    return ws.value, pool.value


def kv_store_init(desc: Desc, workspace, pool, stream=None) -> int:
    h = _vp()
    _check(_lib.hsk_kv_store_init(ctypes.byref(desc), _ptr(workspace), _ptr(pool), _stream(stream), ctypes.byref(h)),
           "hsk_kv_store_init")
    return h.value


def host_rows(store: int, source: int, req: int):
    p, n = _vp(), _i64()
    _check(_lib.hsk_host_rows(store, source, req, ctypes.byref(p), ctypes.byref(n)), "hsk_host_rows")
    return p.value, n.value


def commit_prefill(store: int, stream=None) -> None:
    _check(_lib.hsk_commit_prefill(store, _stream(stream)), "hsk_commit_prefill")


def residency_set(store: int, source: int, req: int, page_ids, stream=None) -> None:
    ids = np.ascontiguousarray(np.asarray(page_ids, dtype=np.int32))
    _check(_lib.hsk_residency_set(store, source, req, _ptr(ids), ids.size, _stream(stream)), "hsk_residency_set")


def reclaim_plan(pages_held, deficit: int) -> int:
    a = np.ascontiguousarray(np.asarray(pages_held, dtype=np.int64))
    q = _i32()
    _check(_lib.hsk_reclaim_plan(_ptr(a), a.size, int(deficit), ctypes.byref(q)), "hsk_reclaim_plan")
    return q.value


def residency_init(store: int, capacity_pages: int, reserve_pages: int, required_pages: int, pages_per_attempt: int,
                   optional: bool = True, stream=None) -> None:
    d = ResidencyDesc(capacity_pages=int(capacity_pages), reserve_pages=int(reserve_pages),
                      required_pages=int(required_pages), pages_per_attempt=int(pages_per_attempt),
                      optional=1 if optional else 0)
    _check(_lib.hsk_residency_init(store, ctypes.byref(d), _stream(stream)), "hsk_residency_init")


def request_admit(store: int, req: int, n_rows: int, history=None, source_stride: int = 0, stream=None,
                  num_requests: int = 0) -> list:
    """Returns the slots reclaimed for the admission; raises HskError(HSK_EWAIT) when it must wait."""
    out = np.zeros(max(1, num_requests), np.int32)
    n = _i32()
    _check(_lib.hsk_request_admit(store, int(req), int(n_rows), _ptr(history), int(source_stride), _stream(stream),
                                  _ptr(out) if num_requests else None, ctypes.byref(n)), "hsk_request_admit")
    return out[:n.value].tolist() if num_requests else []


def request_release(store: int, req: int, stream=None) -> None:
    _check(_lib.hsk_request_release(store, int(req), _stream(stream)), "hsk_request_release")


def residency_reclaim(store: int, deficit: int, num_requests: int, stream=None) -> list:
    out = np.zeros(max(1, num_requests), np.int32)
    n = _i32()
    _check(_lib.hsk_residency_reclaim(store, int(deficit), _stream(stream), _ptr(out), ctypes.byref(n)),
           "hsk_residency_reclaim")
    return out[:n.value].tolist()


def residency_populate(store: int, stream=None, copy_stream=None) -> int:
    n = _i32()
    _check(_lib.hsk_residency_populate(store, _stream(stream), _stream(copy_stream if copy_stream is not None
                                                                      else stream), ctypes.byref(n)),
           "hsk_residency_populate")
    return n.value


def residency_publish(store: int, wait: bool = True, stream=None) -> int:
    n = _i32()
    _check(_lib.hsk_residency_publish(store, _stream(stream), 1 if wait else 0, ctypes.byref(n)),
           "hsk_residency_publish")
    return n.value


def residency_query(store: int) -> dict:
    i = ResidencyInfo()
    _check(_lib.hsk_residency_query(store, ctypes.byref(i)), "hsk_residency_query")
    return {f: getattr(i, f) for f, _ in ResidencyInfo._fields_}


def residency_pages(store: int, req: int, cap: int):
    ids = np.zeros(max(1, cap), np.int32)
    flags = np.zeros(max(1, cap), np.uint8)
    n = _i64()
    _check(_lib.hsk_residency_pages(store, int(req), _ptr(ids), _ptr(flags), int(cap), ctypes.byref(n)),
           "hsk_residency_pages")
    m = min(n.value, cap)
    return ids[:m].copy(), flags[:m].copy()


def resolve_step(store: int, source: int, epoch: int, sel, nq, locs, stats, stream=None) -> None:
    _check(_lib.hsk_resolve_step(store, source, int(epoch), _ptr(sel), _ptr(nq), _ptr(locs), _ptr(stats),
                                 _stream(stream)), "hsk_resolve_step")


def append_rows(store: int, source: int, rows, count: int, stream=None, backup_stream=None) -> None:
    _check(_lib.hsk_append_rows(store, source, _ptr(rows), int(count), _stream(stream),
                                _stream(backup_stream if backup_stream is not None else stream)),
           "hsk_append_rows")


def context_rows(store: int, source: int, req: int) -> int:
    n = _i64()
    _check(_lib.hsk_context_rows(store, source, req, ctypes.byref(n)), "hsk_context_rows")
    return n.value


def completed_rows(n_before: int, n_after: int, m: int):
    first, count = _i64(), _i64()
    _check(_lib.hsk_completed_rows(int(n_before), int(n_after), int(m), ctypes.byref(first), ctypes.byref(count)),
           "hsk_completed_rows")
    return first.value, count.value


def ring_rows(window: int, page_rows: int, k_max: int) -> int:
    n = _i64()
    _check(_lib.hsk_ring_rows(int(window), int(page_rows), int(k_max), ctypes.byref(n)), "hsk_ring_rows")
    return n.value


def ring_write(ring, ring_rows: int, slots: int, rows, count: int, row_bytes: int, t0, stream=None) -> None:
    _check(_lib.hsk_ring_write(_ptr(ring), int(ring_rows), int(slots), _ptr(rows), int(count), int(row_bytes),
                               _ptr(t0), _stream(stream)), "hsk_ring_write")


def ring_window_locs(ring_rows: int, slots: int, window: int, t_end, locs, stream=None) -> None:
    _check(_lib.hsk_ring_window_locs(int(ring_rows), int(slots), int(window), _ptr(t_end), _ptr(locs),
                                     _stream(stream)), "hsk_ring_window_locs")


def replay_plan(store: int, plan_source: int, dst_source: int, stream=None) -> None:
    _check(_lib.hsk_replay_plan(store, plan_source, dst_source, _stream(stream)), "hsk_replay_plan")


_DEDICATED = {}   # device -> torch streams on hardware queues of their own, kept for the life of the process


def dedicated_streams(n: int) -> list:
    """n torch streams, each on a hardware queue of its own (hsk_stream_create), for an overlapped schedule.
    The streams are created on first use and reused by later calls on the same device; they stay alive until the
    process ends, because PyTorch's caching allocator keeps referring to a stream that tensors were allocated on."""
    import torch
    dev = torch.cuda.current_device()
    pool = _DEDICATED.setdefault(dev, [])
    while len(pool) < n:
        h = _vp()
        _check(_lib.hsk_stream_create(ctypes.byref(h)), "hsk_stream_create")
        pool.append(torch.cuda.ExternalStream(h.value))
    return pool[:n]


def release_dedicated_streams() -> None:
    """Destroy the streams dedicated_streams made on the current device, after waiting for them.  Only for callers
    that never allocated a tensor while one of them was the current stream (the caching allocator would keep
    referring to it)."""
    import torch
    pool = _DEDICATED.pop(torch.cuda.current_device(), [])
    for s in pool:
        s.synchronize()
        _check(_lib.hsk_stream_destroy(ctypes.c_void_p(s.cuda_stream)), "hsk_stream_destroy")


def fetch_plan(store: int, source: int, stream=None) -> None:
    _check(_lib.hsk_fetch_plan(store, source, _stream(stream)), "hsk_fetch_plan")


def resolve_fetch_attend(store: int, source: int, epoch: int, sel, nq, locs, stats, adesc, q, out, scratch,
                         scratch_bytes: int, stream=None, copy_stream=None) -> None:
    _check(_lib.hsk_resolve_fetch_attend(store, source, int(epoch), _ptr(sel), _ptr(nq), _ptr(locs), _ptr(stats),
                                         ctypes.byref(adesc), _ptr(q), _ptr(out), _ptr(scratch), int(scratch_bytes),
                                         _stream(stream), _stream(copy_stream if copy_stream is not None else stream)),
           "hsk_resolve_fetch_attend")


def promote_staged(store: int, source: int, locs, nq, accepted, promoted=None, stream=None) -> None:
    _check(_lib.hsk_promote_staged(store, source, _ptr(locs), _ptr(nq), _ptr(accepted), _ptr(promoted),
                                   _stream(stream)), "hsk_promote_staged")


def pool_base(store: int, source: int) -> int:
    p = _vp()
    _check(_lib.hsk_pool_base(store, source, ctypes.byref(p)), "hsk_pool_base")
    return p.value


def attn_scratch_bytes(adesc: AttnDesc) -> int:
    b = ctypes.c_size_t()
    _check(_lib.hsk_attn_scratch_bytes(ctypes.byref(adesc), ctypes.byref(b)), "hsk_attn_scratch_bytes")
    return b.value


def sparse_decode_attn(adesc: AttnDesc, q, pool, locs, nq, out, scratch, scratch_bytes: int, stream=None) -> None:
    _check(_lib.hsk_sparse_decode_attn(ctypes.byref(adesc), _ptr(q), _ptr(pool), _ptr(locs), _ptr(nq), _ptr(out),
                                       _ptr(scratch), int(scratch_bytes), _stream(stream)), "hsk_sparse_decode_attn")


def sparse_decode_attn_noalloc(adesc: AttnDesc, q, pool, locs, nq, out, stream=None) -> None:
    _check(_lib.hsk_sparse_decode_attn_noalloc(ctypes.byref(adesc), _ptr(q), _ptr(pool), _ptr(locs), _ptr(nq),
                                               _ptr(out), _stream(stream)), "hsk_sparse_decode_attn_noalloc")


def resolve_attend(store: int, source: int, epoch: int, sel, locs, stats, adesc: AttnDesc, q, out, scratch,
                   scratch_bytes: int, stream=None) -> None:
    _check(_lib.hsk_resolve_attend(store, source, int(epoch), _ptr(sel), _ptr(locs), _ptr(stats), ctypes.byref(adesc),
                                   _ptr(q), _ptr(out), _ptr(scratch), int(scratch_bytes), _stream(stream)),
           "hsk_resolve_attend")


def snapshot(store: int, source: int, req: int, B: int, n_rows: int, page_rows: int, n_import: int) -> dict:
    """n_rows: the source's context rows now (hsk_context_rows); n_import: ctx_len[req] at creation."""
    key = np.zeros(B, np.int32)
    rec = np.zeros(B, np.uint32)
    order = np.zeros(B, np.uint16)
    pt = np.zeros(max(0, n_rows), np.int32)
    opt = np.zeros(max(1, n_import // page_rows) if page_rows else 1, np.int32)
    _check(_lib.hsk_snapshot(store, source, req, _ptr(key), _ptr(rec), _ptr(order), _ptr(pt), _ptr(opt)),
           "hsk_snapshot")
    return {"key": key, "rec": rec, "order": order.astype(np.int32), "pt": pt,
            "opt": opt if page_rows else np.zeros(0, np.int32)}


def read_plan(store: int, source: int, req: int, cap: int):
    pos = np.zeros(max(cap, 1), np.int32)
    dst = np.zeros(max(cap, 1), np.int32)
    n = _i32()
    _check(_lib.hsk_read_plan(store, source, req, _ptr(pos), _ptr(dst), cap, ctypes.byref(n)), "hsk_read_plan")
    m = min(n.value, cap)
    return pos[:m].copy(), dst[:m].copy()


def sync_status(store: int, stream=None) -> int:
    return int(_lib.hsk_sync_status(store, _stream(stream)))


def kv_store_destroy(store: int) -> None:
    _lib.hsk_kv_store_destroy(store)


# ------------------------------------------------------------------------------------------------ helpers
class KVStore:
    """Owns the device workspace and pool (torch tensors) of one store and the library handle."""

    def __init__(self, *, requests: int, sources: int, row_bytes: int, hot_slots: int, tail_rows: int, ctx,
                 max_ctx: Optional[int] = None, page_rows: int = 0, opt_pool_pages: int = 0, max_queries: int = 1,
                 top_k: int, staging_rows: int = 0, host_alias: bool = False, gather_mode: int = GATHER_ZEROCOPY,
                 gather_blocks: int = 0, staging_arenas: int = 0, device: str = "cuda", stream=None):
        import torch
        self.ctx = np.array(np.broadcast_to(np.asarray(ctx, np.int64), (requests,)))
        self.desc = Desc(num_requests=requests, num_sources=sources, row_bytes=row_bytes, hot_slots=hot_slots,
                         tail_rows=tail_rows, page_rows=page_rows, opt_pool_pages=opt_pool_pages,
                         max_queries=max_queries, top_k=top_k, staging_rows=staging_rows,
                         host_alias_sources=1 if host_alias else 0,
                         max_ctx=int(max_ctx if max_ctx is not None else self.ctx.max()),
                         ctx_len=self.ctx.ctypes.data, gather_mode=gather_mode, gather_blocks=gather_blocks,
                         staging_arenas=staging_arenas)
        ws, pool = workspace_bytes(self.desc)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.pool = torch.empty(pool, dtype=torch.uint8, device=device)
        self.handle = kv_store_init(self.desc, self.workspace, self.pool, stream)
        self.R, self.S, self.B, self.T = requests, sources, hot_slots, tail_rows
        self.row_bytes, self.page_rows, self.max_queries, self.top_k = row_bytes, page_rows, max_queries, top_k
        self.staging_rows, self.opt_pool_pages = staging_rows, opt_pool_pages
        self.staging_arenas = staging_arenas
        self.max_ctx = int(self.desc.max_ctx)
        self.rows_per_source = requests * hot_slots + requests * tail_rows + opt_pool_pages * page_rows + \
            (0 if staging_arenas else requests * staging_rows)

    def host_rows(self, source: int, req: int) -> np.ndarray:
        """The pinned host rows of (source, req) as a writable uint8 array [max_ctx, row_bytes]."""
        p, n = host_rows(self.handle, source, req)
        buf = (ctypes.c_uint8 * (n * self.row_bytes)).from_address(p)
        return np.frombuffer(buf, dtype=np.uint8).reshape(n, self.row_bytes)

    def host_ptr(self, source: int, req: int) -> int:
        return host_rows(self.handle, source, req)[0]

    def commit_prefill(self, stream=None):
        commit_prefill(self.handle, stream)

    def residency_set(self, source: int, req: int, page_ids, stream=None):
        residency_set(self.handle, source, req, page_ids, stream)

    # ---- scheduled residency (Adaptive DHiSparse 3.1) ----
    def residency_init(self, capacity_pages: int, reserve_pages: int, required_pages: int, pages_per_attempt: int,
                       optional: bool = True, stream=None):
        residency_init(self.handle, capacity_pages, reserve_pages, required_pages, pages_per_attempt, optional,
                       stream)
        self.ctx[:] = 0

    def admit(self, req: int, n_rows: int, history=None, source_stride: int = 0, stream=None) -> list:
        out = request_admit(self.handle, req, n_rows, history, source_stride, stream, self.R)
        self.ctx[req] = int(n_rows)
        return out

    def release(self, req: int, stream=None):
        request_release(self.handle, req, stream)
        self.ctx[req] = 0

    def reclaim(self, deficit: int, stream=None) -> list:
        return residency_reclaim(self.handle, deficit, self.R, stream)

    def populate(self, stream=None, copy_stream=None) -> int:
        return residency_populate(self.handle, stream, copy_stream)

    def publish(self, wait: bool = True, stream=None) -> int:
        return residency_publish(self.handle, wait, stream)

    def residency_info(self) -> dict:
        return residency_query(self.handle)

    def residency_pages(self, req: int):
        return residency_pages(self.handle, req, self.max_ctx // self.page_rows if self.page_rows else 0)

    def resolve_step(self, source: int, epoch: int, sel, locs, stats=None, nq=None, stream=None):
        resolve_step(self.handle, source, epoch, sel, nq, locs, stats, stream)

    def promote_staged(self, source: int, locs, accepted, promoted=None, nq=None, stream=None):
        promote_staged(self.handle, source, locs, nq, accepted, promoted, stream)

    def resolve_attend(self, source: int, epoch: int, sel, locs, adesc: AttnDesc, q, out, scratch, stats=None,
                       stream=None):
        resolve_attend(self.handle, source, epoch, sel, locs, stats, adesc, q, out, scratch,
                       scratch.numel() * scratch.element_size(), stream)

    def append_rows(self, source: int, rows, count: int, stream=None, backup_stream=None):
        append_rows(self.handle, source, rows, count, stream, backup_stream)

    def context_rows(self, source: int, req: int) -> int:
        return context_rows(self.handle, source, req)

    def replay_plan(self, plan_source: int, dst_source: int, stream=None):
        replay_plan(self.handle, plan_source, dst_source, stream)

    def fetch_plan(self, source: int, stream=None):
        fetch_plan(self.handle, source, stream)

    def resolve_fetch_attend(self, source: int, epoch: int, sel, locs, adesc, q, out, scratch, stats=None, nq=None,
                             stream=None, copy_stream=None):
        resolve_fetch_attend(self.handle, source, epoch, sel, nq, locs, stats, adesc, q, out, scratch,
                             scratch.numel() * scratch.element_size(), stream, copy_stream)

    def pool_base(self, source: int) -> int:
        return pool_base(self.handle, source)

    def pool_rows(self, source: int):
        """torch uint8 view [rows, row_bytes] from a source's pool base to the end of the pool: the rows its
        locations index (its own region, and the shared staging arenas after the last region)."""
        off = source * self.rows_per_source * self.row_bytes
        return self.pool[off:].view(-1, self.row_bytes)

    def snapshot(self, source: int, req: int) -> dict:
        return snapshot(self.handle, source, req, self.B, self.context_rows(source, req), self.page_rows,
                        int(self.ctx[req]))

    def read_plan(self, source: int, req: int):
        return read_plan(self.handle, source, req, self.max_queries * self.top_k)

    def sync_status(self, stream=None) -> int:
        return sync_status(self.handle, stream)

    def close(self):
        if getattr(self, "handle", None):
            kv_store_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stats_tensor(R: int, device: str = "cuda"):
    import torch
    return torch.zeros(R * STATS_BYTES, dtype=torch.uint8, device=device)


def stats_to_numpy(t) -> np.ndarray:
    return t.cpu().numpy().view(STATS_DTYPE)


def mla_desc(*, requests: int, max_queries: int, heads: int, dk: int, dv: int, top_k: int, row_elems: int,
             scale: float, split: int = 0) -> AttnDesc:
    return AttnDesc(kind=ATTN_MLA, num_requests=requests, max_queries=max_queries, heads=heads, kv_heads=1, dk=dk,
                    dv=dv, top_k=top_k, row_elems=row_elems, page_tokens=1, split=split, scale=scale)


def gqa_desc(*, requests: int, heads: int, kv_heads: int, dh: int, top_k: int, page_tokens: int, scale: float,
             split: int = 0) -> AttnDesc:
    return AttnDesc(kind=ATTN_GQA, num_requests=requests, max_queries=1, heads=heads, kv_heads=kv_heads, dk=dh,
                    dv=dh, top_k=top_k, row_elems=page_tokens * 2 * dh, page_tokens=page_tokens, split=split,
                    scale=scale)
