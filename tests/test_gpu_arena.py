"""GPU tests of the expert arena (pools larger than HBM): the forward through the arena equals
the forward on a pool holding the layer's experts bit for bit (and the oracle on one token),
and every call's hits and misses equal the cache oracle's (oracle/cache.py).  The backing
store is pinned host memory, in both layouts the arena takes: six strided tensors (six copies
per expert) and experts stored whole (one copy each)."""
import sys

import numpy as np
import pytest

import k3x_synth as S
from oracle import cache as C

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_k3x_amd as k3x

    k3x.load_library()
    return torch, k3x


def _backing(torch, k3x, seed, L, E, H, I, whole):
    """Pinned host copies of L layers of E experts.  whole: one buffer, each expert's six
    tensors back to back; else six tensors [L * E][rows][cols]."""
    names = S.TENSOR_NAMES
    if whole:
        eb = k3x.k3x_expert_bytes(H, I)
        buf = torch.empty((L * E, eb), dtype=torch.uint8, pin_memory=True)
        a = buf.numpy()
        for l in range(L):
            for e in range(E):
                ex = S.expert_bytes(seed, l, e, H, I)
                a[l * E + e] = np.concatenate([getattr(ex, n).ravel() for n in names])
        base = buf.data_ptr()
        offs = np.cumsum([0] + [int(np.prod(S.tensor_shape(t, H, I))) for t in range(6)])
        host = {n: base + int(offs[t]) for t, n in enumerate(names)}
        return host, [eb] * 6, [buf]
    tens = {}
    for t, n in enumerate(names):
        rows, cols = S.tensor_shape(t, H, I)
        tens[n] = torch.empty((L * E, rows, cols), dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        hp = S.host_pool(seed, l, E, H, I)
        for n in names:
            tens[n].numpy()[l * E:(l + 1) * E] = hp[n]
    return tens, None, list(tens.values())


@pytest.mark.parametrize("whole", [False, True])
def test_arena_forward_and_policy(dev, orc, whole):
    torch, k3x = dev
    seed, L, E, H, I, slots, k = 77, 2, 32, 256, 384, 20, 6
    _log(f"case: arena, backing {'whole experts' if whole else 'six tensors'}, L={L} E={E} slots={slots}")
    host, strides, keep = _backing(torch, k3x, seed, L, E, H, I, whole)
    arena = k3x.k3x_arena_create(host, slots, L, E, H, I, max_slots_per_call=256,
                                 host_strides=strides)
    pools = [k3x.k3x_expert_pool_create(S.device_pool(seed, l, E, H, I), hidden=H, inter=I,
                                        n_experts=E) for l in range(L)]
    ref = C.SlotCache(slots)
    rng = np.random.default_rng(seed + whole)
    w = 1.0 / np.arange(1, E + 1) ** 1.1
    w /= w.sum()
    cache = {}
    for step in range(40):
        layer, T = step % L, 1 + step % 3
        idx = np.stack([rng.choice(E, k, replace=False, p=w) for _ in range(T)]).astype(np.int32)
        gates = rng.random((T, k)).astype(np.float32)
        gates /= gates.sum(axis=1, keepdims=True)
        x = S.normal_bf16(seed + step, S.P_X, 0, (T, H))
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        idd, gd = torch.from_numpy(idx).cuda(), torch.from_numpy(gates).cuda()
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws = k3x.alloc_workspace(k3x.k3x_moe_workspace_size(arena.pool, T, k))
        hits, misses = k3x.k3x_arena_moe_forward(arena, layer, xd, T, idd, gd, k, y, ws)
        y_ref, _ = k3x.moe_forward(pools[layer], xd, idd, gd)
        torch.cuda.synchronize()
        assert k3x.k3x_fetch_drops(ws) == 0
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), step
        keys = list(dict.fromkeys(int(layer * E + e) for e in idx.ravel()))
        h0, m0 = ref.hits, ref.misses
        ref.serve(keys)
        assert (hits, misses) == (ref.hits - h0, ref.misses - m0), step
        if T == 1:
            y_o = np.zeros((1, H), dtype=np.float32)
            exps = [S.expert_bytes(seed, layer, int(e), H, I) for e in idx[0]]
            d = np.stack([orc.expert_forward(x[0], ex) for ex in exps])[None]
            y_o = orc.combine(gates, d)
            assert np.array_equal(y.cpu().numpy(), y_o), step
    th, tm, tb = k3x.k3x_arena_stats(arena)
    assert (th, tm) == (ref.hits, ref.misses) and tb == tm * k3x.k3x_expert_bytes(H, I)
    _log(f"  hits {th}, misses {tm}")

    # a pinned expert survives every later miss
    slots_, _, _ = k3x.k3x_arena_getmany(arena, 0, [5])
    ref.serve([5])
    k3x.k3x_arena_pin(arena, 0, 5)
    ref.pin(5)
    for e in range(E):
        got, _, _ = k3x.k3x_arena_getmany(arena, 1, [e])
        assert got == ref.serve([E + e])[0]
    got, h, m = k3x.k3x_arena_getmany(arena, 0, [5])
    assert got == slots_ and (h, m) == (1, 0)
    torch.cuda.synchronize()
    arena.close()
    del keep


def test_arena_drops_experts_without_a_slot(dev):
    """More distinct experts in a call than the arena has slots: the experts that get no slot
    (the cache oracle says which) are dropped and counted, and y equals the full pool's
    forward with those slots' ids out of range, bit for bit."""
    torch, k3x = dev
    seed, E, H, I, slots, k = 78, 16, 256, 384, 4, 6
    _log(f"case: arena smaller than a call, E={E} slots={slots} topk={k}")
    host, strides, keep = _backing(torch, k3x, seed, 1, E, H, I, True)
    arena = k3x.k3x_arena_create(host, slots, 1, E, H, I, max_slots_per_call=64,
                                 host_strides=strides)
    pool = k3x.k3x_expert_pool_create(S.device_pool(seed, 0, E, H, I), hidden=H, inter=I,
                                      n_experts=E)
    ref = C.SlotCache(slots)
    rng = np.random.default_rng(seed)
    for step in range(8):
        idx = rng.choice(E, k, replace=False).astype(np.int32)[None]
        gates = rng.random((1, k)).astype(np.float32)
        gates /= gates.sum(axis=1, keepdims=True)
        x = S.normal_bf16(seed + step, S.P_X, 0, (1, H))
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        gd = torch.from_numpy(gates).cuda()
        y = torch.empty((1, H), dtype=torch.float32, device="cuda")
        ws = k3x.alloc_workspace(k3x.k3x_moe_workspace_size(arena.pool, 1, k))
        k3x.k3x_arena_moe_forward(arena, 0, xd, 1, torch.from_numpy(idx).cuda(), gd, k, y, ws)
        keys = [int(e) for e in idx[0]]
        got, _ = ref.serve(keys)
        idx_ref = np.array([[e if s >= 0 else -1 for e, s in zip(keys, got)]], dtype=np.int32)
        n_drop = int((idx_ref < 0).sum())
        assert n_drop >= k - slots, step
        y_ref, _ = k3x.moe_forward(pool, xd, torch.from_numpy(idx_ref).cuda(), gd)
        torch.cuda.synchronize()
        assert k3x.k3x_fetch_drops(ws) == n_drop, step
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), step
    _log(f"  {step + 1} calls, drops checked")
    arena.close()
    del keep
