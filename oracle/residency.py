"""Oracle of the load-adaptive residency scheduler -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", section 3.1:

* Eq. 3: required allocations (hot cache and tail of every admitted request), optional history and the
  admission reserve share the capacity M; required allocations and the reserve come first.
* Only whole pages of the history a request arrived with can be optional; a partly filled page and rows
  produced while decoding never are.
* Eq. 4: an admission that leaves a deficit of D pages reclaims whole requests, walking the admitted ones
  in reclaim order and taking the pages of the first q, q the smallest prefix whose pages cover D; if all
  optional pages together cannot cover D the admission waits and nothing changes.
* Freed capacity is refilled by a round-robin pass over the requests that takes at most a fixed number of
  pages in one attempt; ready locations are tracked apart from allocated pages, so a page whose copy is still in
  flight stays out of the optional map (pending) until it is published.
* Reclaim only after host backing: pages whose rows exist only on the device are backed up first, then
  retired.  Population reserves pages, copies or retains their bytes, then publishes ready locations.
* Resident-first admission: a request whose history arrives on the device keeps complete pages of it as
  optional pages while capacity is spare, with its host backup deferred; the rest goes to host.
* Hence every row of an admitted request's history is at all times ready on the device or backed on host.

Readings where the passage leaves a step open (also listed with the design notes):
* reclaim order: admission order, oldest first;
* round robin: one page per visit, slots visited in index order from a cursor that continues after the
  last slot served; a request's pages in ascending page order; page ids lowest free first;
* a release (request finished) retires its pages without backup: its history is no longer needed;
* a reclaimed request stays admitted and is repopulated later like any other.

The scheduler drives the per-source oracles (:class:`oracle.Source`): ready pages are their optional maps.
"""
from __future__ import annotations

import heapq

import numpy as np

from . import OK, EINVAL, Source

ESTATE = -4
EWAIT = -8

FLAG_READY = 1
FLAG_BACKED = 2


class Residency:
    """Scheduler state over the sources of one store (a request's page g uses the same page id in every
    source's optional pool)."""

    def __init__(self, sources: list[Source], capacity_pages: int, reserve_pages: int, required_pages: int,
                 pages_per_attempt: int, optional: bool = True):
        self.sources = sources
        s0 = sources[0]
        self.R, self.P, self.pool_pages = s0.R, s0.page_rows, s0.opt_pool_pages
        self.M, self.M_res, self.c = int(capacity_pages), int(reserve_pages), int(required_pages)
        self.L = int(pages_per_attempt)
        self.optional = bool(optional) and self.P > 0 and self.pool_pages > 0
        self.admitted = [False] * self.R
        self.seq = [0] * self.R
        self.next_seq = 1
        self.n_import = [0] * self.R
        self.ids: list[list[int]] = [[] for _ in range(self.R)]      # page id or -1
        self.ready: list[list[bool]] = [[] for _ in range(self.R)]
        self.backed: list[list[bool]] = [[] for _ in range(self.R)]
        self.free = list(range(self.pool_pages))
        heapq.heapify(self.free)
        self.cursor = 0

    # ---- Eq. 3 bookkeeping ------------------------------------------------------------------------------
    def required_in_use(self) -> int:
        return self.c * sum(self.admitted)

    def optional_in_use(self) -> int:
        return sum(1 for r in range(self.R) for i in self.ids[r] if i >= 0)

    def free_capacity(self) -> int:
        """Pages optional history may still take under Eq. 3 (never negative)."""
        return self.M - self.M_res - self.required_in_use() - self.optional_in_use()

    # ---- maps of the per-source oracles -------------------------------------------------------------------
    def _publish_maps(self, r: int) -> None:
        n = len(self.ids[r])
        if n == 0:
            return
        m = np.array([self.ids[r][g] if self.ready[r][g] else -1 for g in range(n)], np.int32)
        for s in self.sources:
            assert s.residency_set(r, m) == OK

    def _retire(self, r: int) -> None:
        for g, i in enumerate(self.ids[r]):
            if i >= 0:
                heapq.heappush(self.free, i)
                self.ids[r][g] = -1
                self.ready[r][g] = False
        self._publish_maps(r)

    # ---- section 3.1 operations --------------------------------------------------------------------------
    def reclaim(self, deficit: int) -> tuple[int, list[int]]:
        """Eq. 4 over the admitted requests in admission order: back up, then retire, the pages of the first
        q.  Returns (rc, reclaimed slots); EWAIT and no change when the optional pages cannot cover it."""
        if deficit <= 0:
            return OK, []
        order = sorted((r for r in range(self.R) if self.admitted[r]), key=lambda r: self.seq[r])
        total, q = 0, -1
        for i, r in enumerate(order):
            total += sum(1 for x in self.ids[r] if x >= 0)
            if total >= deficit:
                q = i + 1
                break
        if q < 0:
            return EWAIT, []
        for r in order[:q]:
            for g in range(len(self.ids[r])):        # backup first: device-only rows get a host copy
                if self.ids[r][g] >= 0:
                    self.backed[r][g] = True
            self._retire(r)
        return OK, order[:q]

    def admit(self, r: int, n_rows: int, uid: int, on_device: bool) -> tuple[int, list[int]]:
        """A new request takes free slot r with n_rows of imported history (on the device: resident-first,
        else already on host).  Returns (rc, slots reclaimed for it)."""
        if not (0 <= r < self.R) or n_rows < 1 or n_rows > self.sources[0].max_ctx:
            return EINVAL, []
        if self.admitted[r]:
            return ESTATE, []
        need = self.required_in_use() + self.c + self.optional_in_use() + self.M_res - self.M
        rc, taken = self.reclaim(need)
        if rc != OK:
            return rc, []
        for s in self.sources:
            assert s.admit(r, n_rows, uid) == OK
        self.admitted[r] = True
        self.seq[r] = self.next_seq
        self.next_seq += 1
        self.n_import[r] = int(n_rows)
        npg = n_rows // self.P if self.P else 0
        self.ids[r] = [-1] * npg
        self.ready[r] = [False] * npg
        self.backed[r] = [True] * npg
        if on_device and self.optional:
            for g in range(npg):                      # retain: resident-first, host backup deferred
                if self.free_capacity() <= 0 or not self.free:
                    break
                self.ids[r][g] = heapq.heappop(self.free)
                self.ready[r][g] = True
                self.backed[r][g] = False
            self._publish_maps(r)
        return OK, taken

    def release(self, r: int) -> int:
        """The request in slot r finished: its pages are retired (no backup needed) and the slot is free."""
        if not (0 <= r < self.R):
            return EINVAL
        if not self.admitted[r]:
            return ESTATE
        self._retire(r)
        self.admitted[r] = False
        self.n_import[r] = 0
        self.ids[r], self.ready[r], self.backed[r] = [], [], []
        return OK

    def publish(self) -> int:
        """Pending pages whose copies completed become ready (here: all of them)."""
        n = 0
        for r in range(self.R):
            changed = False
            for g, i in enumerate(self.ids[r]):
                if i >= 0 and not self.ready[r][g]:
                    self.ready[r][g] = True
                    changed = True
                    n += 1
            if changed:
                self._publish_maps(r)
        return n

    def populate(self) -> list[tuple[int, int, int]]:
        """One bounded round-robin attempt: publish completed copies, then reserve up to L pages (they stay
        pending until the next publication).  Returns the (slot, page, id) reserved, in order."""
        self.publish()
        got: list[tuple[int, int, int]] = []
        if not self.optional:
            return got
        r, idle = self.cursor, 0
        while len(got) < self.L and self.free_capacity() > 0 and self.free and idle < self.R:
            g = next((g for g, i in enumerate(self.ids[r]) if i < 0), -1) if self.admitted[r] else -1
            if g >= 0:
                pid = heapq.heappop(self.free)
                self.ids[r][g] = pid
                self.ready[r][g] = False
                got.append((r, g, pid))
                idle = 0
                self.cursor = (r + 1) % self.R
            else:
                idle += 1
            r = (r + 1) % self.R
        return got

    # ---- inspection ------------------------------------------------------------------------------------
    def page_state(self, r: int) -> tuple[np.ndarray, np.ndarray]:
        ids = np.array(self.ids[r], np.int32)
        flags = np.array([(FLAG_READY if self.ready[r][g] else 0) | (FLAG_BACKED if self.backed[r][g] else 0)
                          for g in range(len(self.ids[r]))], np.uint8)
        return ids, flags

    def info(self) -> dict:
        adm = [r for r in range(self.R) if self.admitted[r]]
        ready = sum(1 for r in adm for g, i in enumerate(self.ids[r]) if i >= 0 and self.ready[r][g])
        held = self.optional_in_use()
        return {"admitted": len(adm), "required_pages": self.required_in_use(), "optional_pages": held,
                "ready_pages": ready, "pending_pages": held - ready,
                "unbacked_pages": sum(1 for r in adm for b in self.backed[r] if not b),
                "eligible_pages": sum(len(self.ids[r]) for r in adm), "free_pages": self.free_capacity()}

    def check_invariants(self) -> None:
        """Eq. 3 and the section 3.1 guarantee that every history row is ready on the device or on host."""
        assert self.required_in_use() + self.optional_in_use() + self.M_res <= self.M, "Eq. 3 violated"
        used = [i for r in range(self.R) for i in self.ids[r] if i >= 0]
        assert len(used) == len(set(used)), "a page id is held twice"
        assert not (set(used) & set(self.free)), "a held page id is also free"
        assert len(used) + len(self.free) == self.pool_pages
        for r in range(self.R):
            for g, i in enumerate(self.ids[r]):
                assert (i >= 0 and self.ready[r][g]) or self.backed[r][g], (r, g)
                assert not (self.ready[r][g] and i < 0)
