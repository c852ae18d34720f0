"""Independent brute-force model of one request's KV hierarchy, used to pin the C oracle.

It shares nothing with the oracle but the rules themselves, held in a different representation: the hot
cache is an explicit recency list of slots (least recently used first) that is rebuilt by moving slots to
its end, instead of per-slot timestamps sorted on demand.  Direct rows (tail, ready optional pages) are
found by set membership instead of arithmetic on page ids.

Rules (HiSparse section 3.2 "Replacement policy" and section 3.4; Adaptive DHiSparse section 3.2 and
Figure 2, section 3.3 Eqs. 5-6):
  * tail rows, then ready optional pages, resolve directly and do not touch the hot cache;
  * the other selected rows, taken once each in first-occurrence order over the concatenated query
    lists, are hits when a slot holds them, misses otherwise;
  * victims are the least recently used slots that hold no hit; the i-th miss takes the i-th victim, and
    misses beyond the available slots go to staging;
  * afterwards the filled slots move to the most recent end (lowest slot first), then the hit slots
    (lowest slot first), so hits rank above the same step's fills.
"""
from __future__ import annotations


class BruteRequest:
    def __init__(self, B: int, n: int, T: int = 0, page_rows: int = 0):
        self.B, self.n, self.T, self.page_rows = B, n, T, page_rows
        self.recency = list(range(B))      # least recently used first; never-used slots by slot index
        self.holds = [None] * B            # position held by each slot
        self.ready_pages = {}              # complete page index -> optional page id

    def tail_set(self):
        return set(range(max(0, self.n - self.T), self.n)) if self.T else set()

    def optional_positions(self):
        out = {}
        if not self.page_rows:
            return out
        for g, pid in self.ready_pages.items():
            if pid is None or pid < 0 or (g + 1) * self.page_rows > self.n:
                continue
            for p in range(g * self.page_rows, (g + 1) * self.page_rows):
                out[p] = pid
        return out

    def step(self, lists, staging_rows: int):
        """lists: the request's query lists.  Returns dict with per-selection classes, hit slots,
        misses (in order) with their slot or staging index, evictions, and 'error' for staging
        overflow (state unchanged)."""
        tail = self.tail_set()
        optpos = self.optional_positions()
        flat = [p for lst in lists for p in lst]
        classes = []
        pending_order = []
        seen = set()
        for p in flat:
            if p in tail:
                classes.append("tail")
            elif p in optpos:
                classes.append("opt")
            else:
                classes.append("pending")
                if p not in seen:
                    seen.add(p)
                    pending_order.append(p)
        where = {pos: s for s, pos in enumerate(self.holds) if pos is not None}
        hit_slots = sorted({where[p] for p in pending_order if p in where})
        misses = [p for p in pending_order if p not in where]
        hit_set = set(hit_slots)
        candidates = [s for s in self.recency if s not in hit_set]
        victims = candidates[:len(misses)]
        staged = misses[len(victims):]
        if len(staged) > staging_rows:
            return {"error": "staging"}
        evictions = []
        slot_of_miss = {}
        for p, s in zip(misses, victims):
            if self.holds[s] is not None:
                evictions.append((s, self.holds[s]))
            self.holds[s] = p
            slot_of_miss[p] = s
        staged_at = {p: i for i, p in enumerate(staged)}
        fill_slots = sorted(victims)
        moved = set(fill_slots) | hit_set
        self.recency = [s for s in self.recency if s not in moved] + fill_slots + hit_slots
        self.last_fill, self.last_hit, self.last_staged = list(fill_slots), list(hit_slots), list(staged)
        where = {pos: s for s, pos in enumerate(self.holds) if pos is not None}
        out_cls = []
        for p, c in zip(flat, classes):
            if c != "pending":
                out_cls.append(c)
            elif p in staged_at:
                out_cls.append("staged")
            elif p in slot_of_miss:
                out_cls.append("fill")
            else:
                out_cls.append("hit")
        return {"error": None, "classes": out_cls, "hit_slots": hit_slots, "misses": misses,
                "victims": victims, "staged": staged, "evictions": evictions,
                "slot_of": dict(where)}

    def promote(self, lists, accepted: int):
        """Promotion after the round's acceptance (Adaptive DHiSparse 3.4, Figure 3 callout 3), as read
        here: lists 0..accepted are committed.  Staged rows of the last step that a committed list selected
        (in staging order, skipping rows already held) replace the rows of the last step's touched slots
        that no committed list selected, least recently used first; the slots that received a row rank as
        that step's fills.  Returns the (slot, new position, old position) triples."""
        if not lists:
            return []
        a = min(max(accepted, 0), len(lists) - 1)
        committed = {p for lst in lists[:a + 1] for p in lst}
        held = {pos for pos in self.holds if pos is not None}
        promotable = [p for p in self.last_staged if p in committed and p not in held]
        touched = set(self.last_fill) | set(self.last_hit)
        demotable = [s for s in self.recency if s in touched and self.holds[s] not in committed]
        pairs = []
        for p, s in zip(promotable, demotable):
            pairs.append((s, p, self.holds[s]))
            self.holds[s] = p
        moved = {s for s, _, _ in pairs}
        fills = sorted(set(self.last_fill) | moved)
        hits = sorted(set(self.last_hit) - moved)
        self.recency = [s for s in self.recency if s not in touched] + fills + hits
        self.last_fill, self.last_hit = fills, hits
        return pairs
