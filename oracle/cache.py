"""The routed-expert cache policy, plainly (test infrastructure: only tests/
use it; the library never does).

From "kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM", section
"The cache the project exists for", and "Kimi K3 engine (c/kimi_k3.c)",
section "Streaming design": an LRU of expert slots with pinning; the victim is
found by a linear scan for the least recently used unpinned slot; a slot is an
expert, empty, or in flight (reserved by the batch being prefetched, so the
batch never hands one slot to two reads); a request histogram; a token's
misses fetched as one batch in storage order.

This library's concrete rules, the same ones include/k3g.h states: a step's
distinct experts are taken in ascending id (storage order); hits are refreshed
first and are not victims of the step; a miss takes the first empty slot, else
the unpinned slot with the oldest last use among those the step neither uses
nor fills (equal ages: the lower slot); a step whose misses do not fit the
available slots is refused with nothing changed.
"""
from __future__ import annotations

EMPTY = "empty"
INFLIGHT = "inflight"


class CacheRefused(Exception):
    pass


class LruSlots:
    def __init__(self, n_slots: int, n_total: int):
        self.state = [EMPTY] * n_slots          # EMPTY, INFLIGHT or an expert id
        self.receiving = [None] * n_slots       # the expert an in-flight slot receives
        self.age = [-1] * n_slots               # step of the last use
        self.where = {}                         # expert -> slot
        self.pinned = set()
        self.hist = [0] * n_total
        self.step = 0
        self.hits = self.misses = self.evictions = 0

    def finish_batch(self):
        for s, st in enumerate(self.state):
            if st == INFLIGHT:
                self.state[s] = self.receiving[s]
                self.receiving[s] = None

    def request(self, idx):
        """One step: idx is a list of token rows of expert ids (-1 = dropped).
        Returns (slot rows, [(expert, slot) copies in order])."""
        self.finish_batch()
        wanted = sorted({e for row in idx for e in row if e >= 0})
        used = {self.where[e] for e in wanted if e in self.where}
        n_miss = sum(1 for e in wanted if e not in self.where)
        available = [s for s, st in enumerate(self.state)
                     if s not in used and (st == EMPTY or (st != INFLIGHT and st not in self.pinned))]
        if n_miss > len(available):
            raise CacheRefused(f"{n_miss} misses, {len(available)} slots")
        self.step += 1
        for row in idx:
            for e in row:
                if e >= 0:
                    self.hist[e] += 1
        for e in wanted:
            if e in self.where:
                self.age[self.where[e]] = self.step
                self.hits += 1
        copies = []
        for e in wanted:
            if e in self.where:
                continue
            empties = [s for s, st in enumerate(self.state) if st == EMPTY]
            if empties:
                s = empties[0]
            else:
                cands = [s for s, st in enumerate(self.state)
                         if s not in used and st != INFLIGHT and st not in self.pinned]
                s = min(cands, key=lambda i: (self.age[i], i))
                del self.where[self.state[s]]
                self.evictions += 1
            self.state[s] = INFLIGHT
            self.receiving[s] = e
            self.where[e] = s
            self.age[s] = self.step
            used.add(s)
            copies.append((e, s))
            self.misses += 1
        slots = [[self.where[e] if e >= 0 else -1 for e in row] for row in idx]
        return slots, copies
