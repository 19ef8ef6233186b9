"""Oracle of the expert cache (test infrastructure only: tests/, smoke() and bench.py's
cpu_baseline use it; the product path never does).

Written from kimi-k3-in-c README, Part II section 12 "An LRU cache for the experts" and
section 13 "How big should that cache be? Ask the trace":

  - A slot holds an expert key, or is EMPTY, or INFLIGHT (reserved, being filled).  The victim
    for a miss is the first EMPTY slot, else the least recently used slot that is neither
    INFLIGHT nor pinned; none means the request cannot be cached.
  - A batch of requests (one token's experts) is served in three phases: reserve serially
    (a resident key is a hit; a miss takes a victim and marks it INFLIGHT), fetch the misses
    (in the backing store's offset order), publish each fetched key in its slot.
  - Trace replay: the hit rate of LRU, of Belady's rule (evict the resident key needed
    furthest in the future -- a ceiling, not a policy) and of LRU with some keys pinned, as a
    function of the number of slots.

Readings (where the pages leave a step open): a request touches its key at one global tick
per request, in request order; a batch's hits and reservations are protected from eviction
by its later misses (a batch never evicts an expert it still needs); each fetched key is
published in the slot reserved for it; PIN+LRU pins the keys given by the caller (the replay
pins the most requested keys of the trace).  Plain Python loops, meant for traces of up to a
few hundred thousand requests.
"""
from __future__ import annotations

import heapq
from collections import defaultdict

EMPTY = -1
INFLIGHT = -2


def lru_hits(trace, cap, pinned=()):
    """Hits of LRU with cap slots over the trace (a sequence of hashable keys).  Keys in
    `pinned` are never evicted once resident (they still take a slot)."""
    pinned = set(pinned)
    last = {}       # resident key -> tick of its last use
    hits = 0
    for tick, k in enumerate(trace):
        if k in last:
            hits += 1
            last[k] = tick
            continue
        if cap <= 0:
            continue
        if len(last) >= cap:
            cands = [r for r in last if r not in pinned]
            if not cands:
                continue  # every slot pinned: the request is not cached
            victim = min(cands, key=lambda r: last[r])
            del last[victim]
        last[k] = tick
    return hits


def belady_hits(trace, cap):
    """Hits of Belady's rule: on a miss with every slot taken, evict the resident key whose
    next request lies furthest ahead (a key never requested again is furthest of all).

    One backward pass finds, for every request, the position of the same key's next request.
    Resident keys are kept with that position, and a max-heap orders them by it; a heap entry
    whose key has been requested again (or evicted) since it was pushed no longer matches the
    key's recorded position and is discarded when it reaches the top."""
    n = len(trace)
    later = [n] * n  # n: never requested again
    upcoming = {}
    for i in range(n - 1, -1, -1):
        later[i] = upcoming.get(trace[i], n)
        upcoming[trace[i]] = i
    due = {}   # resident key -> position of its next request
    heap = []  # (-next request, push order, key): the push order keeps keys from being compared
    hits = 0
    for i, k in enumerate(trace):
        if k in due:
            hits += 1
        elif cap <= 0:
            continue
        elif len(due) >= cap:
            while True:
                neg_next, _, v = heapq.heappop(heap)
                if due.get(v) == -neg_next:
                    break
            del due[v]
        due[k] = later[i]
        heapq.heappush(heap, (-later[i], i, k))
    return hits


def most_requested(trace, n):
    """The n most requested keys of the trace (ties: the smaller key first)."""
    count = defaultdict(int)
    for k in trace:
        count[k] += 1
    order = sorted(count, key=lambda k: (-count[k], k))
    return order[:n]


class SlotCache:
    """The three-state slot cache, batch by batch: serve(keys) returns the slot of each key,
    with -1 for a key that could not be given a slot, and records which keys were fetched."""

    def __init__(self, n_slots):
        self.key = [EMPTY] * n_slots
        self.used = [0] * n_slots
        self.pinned = [False] * n_slots
        self.tick = 0
        self.hits = 0
        self.misses = 0

    def lookup(self, k):
        for s, kk in enumerate(self.key):
            if kk == k:
                return s
        return -1

    def pick_victim(self, protected):
        best, oldest = -1, None
        for s, kk in enumerate(self.key):
            if kk == INFLIGHT or s in protected:
                continue
            if kk == EMPTY:
                return s
            if self.pinned[s]:
                continue
            if oldest is None or self.used[s] < oldest:
                best, oldest = s, self.used[s]
        return best

    def serve(self, keys, order_key=None):
        """One batch.  Returns (slots, fetched): slots[j] for keys[j]; fetched = the
        (key, slot) pairs filled from the backing store, in fetch order (by order_key of the
        key, default the key itself)."""
        slots = [-1] * len(keys)
        protected = set()
        reserve = []
        for j, k in enumerate(keys):
            s = self.lookup(k)
            if s < 0:  # a key already reserved by this batch shares that slot
                for jj in range(j):
                    if keys[jj] == k and slots[jj] >= 0:
                        s = slots[jj]
                        break
            if s >= 0:
                if self.key[s] != INFLIGHT:
                    self.hits += 1
                    self.tick += 1
                    self.used[s] = self.tick
                slots[j] = s
                protected.add(s)
                continue
            s = self.pick_victim(protected)
            if s < 0:
                continue
            self.misses += 1
            self.key[s] = INFLIGHT
            self.tick += 1
            self.used[s] = self.tick
            slots[j] = s
            protected.add(s)
            reserve.append((k, s))
        ok = order_key or (lambda k: k)
        fetched = sorted(reserve, key=lambda ks: ok(ks[0]))
        for k, s in fetched:
            self.key[s] = k
        return slots, fetched

    def pin(self, k):
        s = self.lookup(k)
        if s >= 0:
            self.pinned[s] = True
        return s
