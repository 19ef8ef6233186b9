"""Pins of the expert-cache oracle (oracle/cache.py) against what the definitions and the
textbook fix: published fault counts, the stack-distance characterisation of LRU, exhaustive
search for the optimal replacement on tiny traces, and the slot rules of the pages' cache
(kimi-k3-in-c README, Part II sections 12 and 13)."""
import itertools

import numpy as np
import pytest

from oracle import cache as C

# The reference string of the classic page-replacement example (Silberschatz, Galvin and
# Gagne, "Operating System Concepts", section 10.4): with 3 frames, FIFO takes 15 faults,
# the optimal rule 9 and LRU 12.
REF = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]


def test_textbook_fault_counts():
    assert len(REF) - C.lru_hits(REF, 3) == 12
    assert len(REF) - C.belady_hits(REF, 3) == 9


def _stack_distance_hits(trace, cap):
    """LRU hits from its characterisation: a request hits iff fewer than cap distinct keys
    were requested since the key's previous request."""
    hits = 0
    for i, k in enumerate(trace):
        prev = max((j for j in range(i) if trace[j] == k), default=None)
        if prev is None:
            continue
        if len(set(trace[prev + 1:i])) < cap:
            hits += 1
    return hits


def _zipf_trace(seed, n, keys, s=1.1):
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, keys + 1) ** s
    return list(rng.choice(keys, size=n, p=w / w.sum()))


@pytest.mark.parametrize("cap", [1, 2, 5, 17])
def test_lru_equals_stack_distance(cap):
    t = _zipf_trace(cap, 400, 40)
    assert C.lru_hits(t, cap) == _stack_distance_hits(t, cap)


def _best_hits(trace, cap):
    """Exhaustive search over every eviction choice (tiny traces only)."""
    best = 0

    def go(i, res, hits):
        nonlocal best
        if i == len(trace):
            best = max(best, hits)
            return
        k = trace[i]
        if k in res:
            go(i + 1, res, hits + 1)
        elif len(res) < cap:
            go(i + 1, res | {k}, hits)
        else:
            for v in res:
                go(i + 1, (res - {v}) | {k}, hits)

    go(0, frozenset(), 0)
    return best


def test_belady_is_optimal_on_tiny_traces():
    rng = np.random.default_rng(1)
    for _ in range(40):
        n, keys, cap = int(rng.integers(4, 11)), int(rng.integers(2, 5)), int(rng.integers(1, 3))
        t = list(rng.integers(0, keys, n))
        assert C.belady_hits(t, cap) == _best_hits(t, cap), (t, cap)


def test_bounds_and_monotonicity():
    t = _zipf_trace(7, 2000, 300)
    distinct = len(set(t))
    prev_l = prev_b = -1
    for cap in (1, 4, 16, 64, 256, 300, 400):
        l, b = C.lru_hits(t, cap), C.belady_hits(t, cap)
        assert l <= b <= len(t) - distinct  # compulsory misses bound every rule
        assert l >= prev_l and b >= prev_b  # both have the inclusion property
        prev_l, prev_b = l, b
    assert C.lru_hits(t, distinct) == C.belady_hits(t, distinct) == len(t) - distinct


def test_pinned_keys_are_never_evicted():
    # LRU alone evicts key 1 (the oldest) when 3 arrives; pinned, key 2 goes instead
    t = [1, 2, 3, 1, 2]
    assert C.lru_hits(t, 2) == 0
    assert C.lru_hits(t, 2, pinned={1}) == 1
    assert C.most_requested([5, 3, 5, 3, 9, 3], 2) == [3, 5]


def test_slot_cache_victim_rules():
    c = C.SlotCache(3)
    slots, fetched = c.serve([10, 11])
    assert slots == [0, 1] and fetched == [(10, 0), (11, 1)]  # EMPTY slots first, in order
    slots, fetched = c.serve([12])
    assert slots == [2]  # the last EMPTY slot
    c.serve([10])  # 10 becomes the most recent; 11 is now the least recent
    slots, fetched = c.serve([13])
    assert slots == [1] and fetched == [(13, 1)]
    c.pin(12)  # 12 is now the least recent but pinned: 10 goes
    slots, _ = c.serve([14])
    assert slots == [0]
    assert (c.hits, c.misses) == (1, 5)


def test_slot_cache_protects_the_batch_and_orders_fetches():
    c = C.SlotCache(2)
    c.serve([1, 2])
    # 1 is a hit of this batch; the miss of 3 must not evict it (2 goes), and the miss of 4
    # finds every slot protected: it gets no slot
    slots, fetched = c.serve([1, 3, 4])
    assert slots == [0, 1, -1] and fetched == [(3, 1)]
    # fetches run in backing-store order, whatever the request order
    c2 = C.SlotCache(4)
    _, fetched = c2.serve([9, 2, 7], order_key=lambda k: k)
    assert [k for k, _ in fetched] == [2, 7, 9]


def test_slot_cache_matches_sequential_lru_when_the_batch_fits():
    rng = np.random.default_rng(4)
    for cap, k in ((24, 8), (40, 16)):
        t = _zipf_trace(cap, 60 * k, 96)
        batches = []
        for i in range(0, len(t), k):  # distinct keys per batch, as a router picks them
            b = list(dict.fromkeys(t[i:i + k]))
            batches.append(b)
        flat = list(itertools.chain.from_iterable(batches))
        c = C.SlotCache(cap)
        for b in batches:
            c.serve(b)
        assert c.hits == C.lru_hits(flat, cap), (cap, k)
        assert c.hits + c.misses == len(flat)
