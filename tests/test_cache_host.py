"""The library's expert-cache policy and trace replay (host code, no GPU) against the cache
oracle (oracle/cache.py), and the arena's host-side argument checks."""
import ctypes

import numpy as np
import pytest

from oracle import cache as C


@pytest.fixture(scope="module")
def k3x():
    import mxfp4_routed_expert_k3x_amd as k3x

    k3x.load_library()
    return k3x


def _zipf(seed, n, keys, s=1.1):
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, keys + 1) ** s
    return [int(v) for v in rng.choice(keys, size=n, p=w / w.sum())]


def test_replay_textbook(k3x):
    ref = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]
    assert k3x.k3x_cache_replay(ref, 3, k3x.K3X_CACHE_LRU) == 8
    assert k3x.k3x_cache_replay(ref, 3, k3x.K3X_CACHE_BELADY) == 11


@pytest.mark.parametrize("cap", [0, 1, 3, 16, 64, 250])
def test_replay_equals_oracle(k3x, cap):
    t = _zipf(cap + 1, 5000, 300)
    assert k3x.k3x_cache_replay(t, cap, k3x.K3X_CACHE_LRU) == C.lru_hits(t, cap)
    assert k3x.k3x_cache_replay(t, cap, k3x.K3X_CACHE_BELADY) == C.belady_hits(t, cap)
    pins = C.most_requested(t, cap // 2)
    assert k3x.k3x_cache_replay(t, cap, k3x.K3X_CACHE_PIN_LRU, pins) == C.lru_hits(t, cap, pins)


def test_replay_rejects_bad_arguments(k3x):
    lib = k3x.lib()
    h = ctypes.c_int64()
    t = (ctypes.c_int64 * 3)(1, 2, 3)
    assert lib.k3x_cache_replay(t, 3, 2, 7, None, 0, ctypes.byref(h)) == k3x.K3X_E_INVALID_ARG
    assert lib.k3x_cache_replay(t, 3, -1, 0, None, 0, ctypes.byref(h)) == k3x.K3X_E_INVALID_ARG
    assert lib.k3x_cache_replay(None, 3, 2, 0, None, 0, ctypes.byref(h)) == k3x.K3X_E_INVALID_ARG
    assert lib.k3x_cache_replay(t, 3, 2, 2, None, 4, ctypes.byref(h)) == k3x.K3X_E_INVALID_ARG


@pytest.mark.parametrize("cap,k", [(24, 8), (40, 16), (10, 16), (6, 4)])
def test_batched_policy_equals_oracle_slot_by_slot(k3x, cap, k):
    """The arena's policy, batch by batch: every slot it gives equals the oracle's, also when
    the batch is larger than the cache (its later misses get no slot)."""
    t = _zipf(cap * 7 + k, 80 * k, 120)
    batches = [list(dict.fromkeys(t[i:i + k])) for i in range(0, len(t), k)]
    got = k3x.k3x_cache_replay_batches(batches, cap)
    o = C.SlotCache(cap)
    for b, g in zip(batches, got):
        slots, _ = o.serve(b)
        assert g == slots, (b, g, slots)


def test_batched_policy_repeated_key_shares_its_slot(k3x):
    got = k3x.k3x_cache_replay_batches([[3, 5, 3], [5, 9]], 4)
    o = C.SlotCache(4)
    assert got == [o.serve([3, 5, 3])[0], o.serve([5, 9])[0]]
    assert got[0][0] == got[0][2]


def test_arena_create_checks(k3x):
    lib = k3x.lib()
    fake = 1 << 40

    def desc(**kw):
        d = k3x.k3x_arena_desc()
        d.n_slots, d.n_layers, d.n_experts = 8, 2, 16
        d.hidden, d.inter, d.group = 256, 384, 32
        for i in range(6):
            d.host[i] = fake + i * (1 << 30)
        d.max_slots_per_call = 64
        for kk, v in kw.items():
            setattr(d, kk, v)
        return d

    h = ctypes.c_void_p()
    for kw, want in (({"n_slots": 0}, k3x.K3X_E_INVALID_ARG), ({"n_slots": 9000}, k3x.K3X_E_INVALID_ARG),
                     ({"n_layers": 0}, k3x.K3X_E_INVALID_ARG), ({"max_slots_per_call": 0}, k3x.K3X_E_INVALID_ARG),
                     ({"group": 16}, k3x.K3X_E_UNSUPPORTED), ({"hidden": 200}, k3x.K3X_E_UNSUPPORTED)):
        assert lib.k3x_arena_create(ctypes.byref(desc(**kw)), ctypes.byref(h)) == want, kw
        assert h.value is None
    d = desc()
    d.host[3] = None
    assert lib.k3x_arena_create(ctypes.byref(d), ctypes.byref(h)) == k3x.K3X_E_INVALID_ARG
    d = desc()
    d.host_stride[0] = 100  # below the dense size of w1_packed
    assert lib.k3x_arena_create(ctypes.byref(d), ctypes.byref(h)) == k3x.K3X_E_INVALID_ARG
    assert k3x.k3x_expert_bytes(3584, 3072) == 17547264
