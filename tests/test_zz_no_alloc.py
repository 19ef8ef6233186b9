"""The expert forward that allocates nothing (k3x_moe_forward_noalloc, the library's built-in
scratch as its workspace) against k3x_moe_forward with a caller's workspace: the same kernels,
so the outputs are equal bit for bit, on consecutive calls that reuse the scratch (the second
smaller than the first), on every path; the drop count reaches the caller's device int64; a
call too large for the scratch is refused before anything is enqueued."""
import sys

import numpy as np
import pytest

import k3x_synth as S

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


def _t(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _both(torch, k3x, pool, x, idx, gates, k):
    """Runs both entry points on the same inputs; returns (y_noalloc, drops_noalloc, y_ws,
    drops_ws)."""
    T, H = x.shape[0], pool.H
    y_na = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    drops = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    k3x.k3x_moe_forward_noalloc(pool, x, T, idx, gates, k, y_na, drops)
    y_ws = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = k3x.alloc_workspace(k3x.k3x_moe_workspace_size(pool, T, k))
    k3x.k3x_moe_forward(pool, x, T, idx, gates, k, y_ws, ws)
    torch.cuda.synchronize()
    return y_na, int(drops.item()), y_ws, k3x.k3x_fetch_drops(ws)


@pytest.mark.parametrize("E,H,I,calls", [
    (8, 512, 1024, [(40, 2), (1, 4)]),    # sorted-tile path, then exact decode
    (6, 384, 256, [(9, 3), (3, 2)]),      # grouped path twice
    (896, 3584, 3072, [(32, 16), (1, 16)]),  # the K3 shape: a 32-token batch, then one token
])
def test_noalloc_equals_workspace_forward(dev, E, H, I, calls):
    torch, k3x = dev
    seed = 6000 + E + H + I
    pool = k3x.k3x_expert_pool_create(S.device_pool(seed, 0, E, H, I), hidden=H, inter=I,
                                      n_experts=E)
    for n, (T, k) in enumerate(calls):
        _log(f"case: noalloc E={E} H={H} I={I} call {n}: T={T} k={k}")
        x = _t(torch, S.normal_bf16(seed + n, S.P_X, 0, (T, H)))
        i_, g_ = S.uniform_routing(seed + n, T, E, k)
        if n == 0 and T > 1:
            i_[T - 1, k - 1] = E + 5  # one dropped slot in the first call
        idx, gates = _t(torch, i_), _t(torch, g_)
        y_na, d_na, y_ws, d_ws = _both(torch, k3x, pool, x, idx, gates, k)
        assert torch.equal(y_na.view(torch.int32), y_ws.view(torch.int32)), (T, k)
        assert d_na == d_ws == (1 if n == 0 and T > 1 else 0)
    pool.close()


def test_noalloc_refuses_calls_larger_than_its_scratch(dev):
    torch, k3x = dev
    _log("case: noalloc refusal")
    H, I = 3584, 3072
    pool = k3x.k3x_expert_pool_create(S.device_pool(7, 0, 4, H, I), hidden=H, inter=I,
                                      n_experts=4)
    T = 103
    assert k3x.k3x_moe_workspace_size(pool, T, 16) > k3x.K3X_NOALLOC_SCRATCH_BYTES
    y = torch.full((T, H), 1.5, dtype=torch.float32, device="cuda")
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    idx = torch.zeros((T, 16), dtype=torch.int32, device="cuda")
    g = torch.zeros((T, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        k3x.k3x_moe_forward_noalloc(pool, x, T, idx, g, 16, y)
    torch.cuda.synchronize()
    assert torch.all(y == 1.5)  # nothing was enqueued
    pool.close()
