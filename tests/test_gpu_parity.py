"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Routing indices must equal the oracle's element by element and gates bit for bit; y must
reach relative L2 <= 1e-4 and max-abs <= 1e-3 * max|y_ref| (tests/cases.py).  Inputs are
seeded (k3x_synth); expected values come from the oracle only.
"""
import sys

import numpy as np
import pytest

import k3x_synth as S
from cases import (assert_y_close, assert_y_close_oracle, oracle_forward_all, oracle_forward_sampled,
                   token_errors, y_errors)

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


def _np(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def _pool(torch, k3x, dev_tensors, E, H, I, act="swiglu"):
    if act == "swiglu":
        return k3x.k3x_expert_pool_create(dev_tensors, hidden=H, inter=I, n_experts=E)
    _, b1, b2 = act
    return k3x.k3x_expert_pool_create(dev_tensors, hidden=H, inter=I, n_experts=E,
                                      activation="situ", situ_b1=b1, situ_b2=b2)


SITU = ("situ", 4.0, 25.0)


# ------------------------------------------------------------------------------------------
# generator twin
# ------------------------------------------------------------------------------------------
def test_synth_device_bytes_equal_host_bytes(dev):
    torch, _ = dev
    _log("case: synth device vs host, E=3 H=256 I=384")
    E, H, I = 3, 256, 384
    d = S.device_pool(99, 2, E, H, I)
    h = S.host_pool(99, 2, E, H, I)
    for n in S.TENSOR_NAMES:
        assert np.array_equal(_np(d[n]), h[n]), n
    _log("case: synth device vs host, sampled windows of full-size experts")
    big = S.device_pool(7, 1, 4, S.H_K3, S.I_K3)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for t, n in enumerate(S.TENSOR_NAMES):
        arr = _np(big[n]).reshape(4, -1)
        for _ in range(3):
            e = int(rng.integers(0, 4))
            b0 = int(rng.integers(0, arr.shape[1] - 64))
            if t % 2 == 0:
                want = S.packed_bytes(7, 1, e, t, 64, b0=b0)
            else:
                want = S.scale_bytes(7, 1, e, t, 64, s0=b0)
            assert np.array_equal(arr[e, b0:b0 + 64], want), (n, e, b0)


# ------------------------------------------------------------------------------------------
# expert forward, small shapes (several tiles, ragged tails, duplicates, drops)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("E,H,I,T,k", [(8, 256, 384, 5, 3), (6, 128, 128, 7, 5), (16, 384, 256, 40, 4)])
def test_moe_small_parity(dev, orc, E, H, I, T, k):
    torch, k3x = dev
    _log(f"case: moe small E={E} H={H} I={I} T={T} k={k}")
    seed = 1000 + E + H + I + T
    host = S.host_pool(seed, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(seed, 0, E, H, I), E, H, I)
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    idx, gates = S.uniform_routing(seed, T, E, k)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    y_ref, drops = orc.moe_forward(host, x, idx, gates)
    assert drops == 0
    assert_y_close(_np(y), y_ref, f"E={E} H={H} I={I} T={T} k={k}")


@pytest.mark.parametrize("E,H,I,T,k", [(4, 512, 512, 40, 2), (2, 512, 1536, 300, 1),
                                       (3, 1536, 1024, 100, 2), (8, 1024, 512, 200, 3),
                                       (64, 512, 512, 3, 4), (16, 1024, 512, 2, 8)])
def test_prefill_path_parity(dev, orc, E, H, I, T, k):
    """Batches of two or more tokens take the sorted-tile kernels (tiles of up to 96 slots,
    items of 256 h rows and 512 d rows): several tiles per expert, ragged last tiles, several
    row chunks per tile, K loops of every length modulo the three-stage weight ring."""
    torch, k3x = dev
    _log(f"case: prefill path E={E} H={H} I={I} T={T} k={k}")
    seed = 2000 + E + H + I + T
    host = S.host_pool(seed, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(seed, 0, E, H, I), E, H, I)
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)  # duplicates allowed
    if T > 100:
        idx[7, 0] = -5  # a dropped slot
    _, gates = S.uniform_routing(seed, T, k, k)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    y_ref, drops = orc.moe_forward(host, x, idx, gates)
    assert k3x.k3x_fetch_drops(ws) == drops
    r = assert_y_close_oracle(_np(y), y_ref, lambda: orc.moe_forward(host, x, idx, gates, acc="f64")[0],
                              f"prefill E={E} H={H} I={I} T={T} k={k}")
    _log(f"  rel_l2={r[0]:.3e} max_abs={r[1]:.3e}")


def test_moe_duplicates_and_drops(dev, orc):
    torch, k3x = dev
    E, H, I, T, k = 6, 256, 256, 9, 6
    _log(f"case: moe duplicates and drops E={E} T={T} k={k}")
    host = S.host_pool(5, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(5, 0, E, H, I), E, H, I)
    x = S.normal_bf16(5, S.P_X, 0, (T, H))
    rng = np.random.default_rng(5)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)  # duplicates within tokens
    idx[0, 0] = -1
    idx[3, 5] = E
    idx[8, 2] = 1 << 30
    _, gates = S.uniform_routing(5, T, k, k)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 3
    y_ref, drops = orc.moe_forward(host, x, idx, gates)
    assert drops == 3
    assert_y_close(_np(y), y_ref, "duplicates/drops")
    # the next call resets the counter
    idx2 = np.clip(idx, 0, E - 1).astype(np.int32)
    k3x.moe_forward(pool, _t(torch, x), _t(torch, idx2), _t(torch, gates), ws=ws)
    assert k3x.k3x_fetch_drops(ws) == 0


@pytest.mark.parametrize("H,I,E,k", [(512, 384, 12, 1), (512, 384, 12, 9), (2560, 2304, 12, 17),
                                       (2560, 2304, 12, 40), (512, 384, 12, 64),
                                       (768, 2176, 6, 5), (512, 3072, 6, 16)])
def test_decode_exact_slot_counts(dev, orc, H, I, E, k):
    """Single-token decode with 1 to 64 slots (duplicates and one dropped slot when k > 1):
    every workgroup of the W2 + combine launch takes several slots per wave, and the
    result equals the fp32 oracle's bit for bit.  W2 rows of 65 to 96 groups (I = 2176,
    2304, 3072) share the load of their second halves two rows at a time, including an odd
    number of rows per workgroup (H = 768: three)."""
    torch, k3x = dev
    _log(f"case: exact decode H={H} I={I} E={E} k={k}")
    host = S.host_pool(11, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(11, 0, E, H, I), E, H, I)
    x = S.normal_bf16(11, S.P_X, 0, (1, H))
    rng = np.random.default_rng(k)
    idx = rng.integers(0, E, (1, k)).astype(np.int32)
    if k > 1:
        idx[0, k // 2] = -1
    _, gates = S.uniform_routing(11, 1, k, k)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    y_ref, drops = orc.moe_forward(host, x, idx, gates)
    assert k3x.k3x_fetch_drops(ws) == drops == (1 if k > 1 else 0)
    assert np.array_equal(_np(y), y_ref)


@pytest.mark.parametrize("T,H,I,E,k", [(1030, 256, 256, 6, 8), (1100, 512, 512, 40, 8)])
def test_moe_split_sort(dev, orc, T, H, I, E, k):
    """Batches of 8192 slots or more are sorted in slices (count, scan, scatter): duplicates
    within tokens, out-of-range ids counted as drops, on the grouped path (H = 256) and the
    prefill path (H = 512)."""
    torch, k3x = dev
    _log(f"case: split sort T={T} H={H} I={I} E={E} k={k}")
    host = S.host_pool(17, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(17, 0, E, H, I), E, H, I)
    x = S.normal_bf16(17, S.P_X, 0, (T, H))
    rng = np.random.default_rng(T)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[5, 3] = -1
    idx[700, 0] = E
    idx[T - 1, k - 1] = 1 << 20
    _, gates = S.uniform_routing(17, T, k, k)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 3
    y_ref, drops = orc.moe_forward(host, x, idx, gates)
    assert drops == 3
    assert_y_close(_np(y), y_ref, "split sort")


def test_strided_pool(dev, orc):
    """Experts laid out with padding between them (per-tensor byte strides larger than the
    dense size, as when experts sit inside a bigger arena): single-token decode stays
    bit-exact and the multi-token paths match the oracle."""
    torch, k3x = dev
    E, H, I = 6, 512, 512
    _log(f"case: strided pool E={E} H={H} I={I}")
    host = S.host_pool(23, 0, E, H, I)
    dense = S.device_pool(23, 0, E, H, I)
    tensors, strides = {}, []
    for t, name in enumerate(S.TENSOR_NAMES):
        per = dense[name][0].numel()
        stride = per + 256 * (t + 1)  # every stride a multiple of 16, all different
        buf = torch.full((E * stride,), 0xA5, dtype=torch.uint8, device="cuda")
        for e in range(E):
            buf[e * stride:e * stride + per] = dense[name][e].reshape(-1)
        tensors[name] = buf
        strides.append(stride)
    pool = k3x.k3x_expert_pool_create(tensors, hidden=H, inter=I, n_experts=E, strides=strides)
    for T, k in ((1, 4), (9, 3), (40, 2)):
        x = S.normal_bf16(23 + T, S.P_X, 0, (T, H))
        rng = np.random.default_rng(T)
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        _, gates = S.uniform_routing(23 + T, T, k, k)
        y, _ = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
        torch.cuda.synchronize()
        y_ref, _ = orc.moe_forward(host, x, idx, gates)
        if T == 1:
            assert np.array_equal(_np(y), y_ref)
        else:
            assert_y_close_oracle(_np(y), y_ref,
                                  lambda: orc.moe_forward(host, x, idx, gates, acc="f64")[0],
                                  f"strided pool T={T}")


def test_largest_rows(dev, orc):
    """Rows of 128 groups (H = I = 4096, the largest the exact decode kernel and the LDS
    scale buffer of the sorted-tile kernels take): decode bit-exact, prefill path within
    tolerance."""
    torch, k3x = dev
    E, H, I = 6, 4096, 4096
    _log(f"case: largest rows E={E} H={H} I={I}")
    host = S.host_pool(29, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(29, 0, E, H, I), E, H, I)
    for T, k in ((1, 6), (24, 2)):
        x = S.normal_bf16(29 + T, S.P_X, 0, (T, H))
        rng = np.random.default_rng(29 + T)
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        _, gates = S.uniform_routing(29 + T, T, k, k)
        y, _ = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
        torch.cuda.synchronize()
        y_ref, _ = orc.moe_forward(host, x, idx, gates)
        if T == 1:
            assert np.array_equal(_np(y), y_ref)
        else:
            r = assert_y_close_oracle(_np(y), y_ref,
                                      lambda: orc.moe_forward(host, x, idx, gates, acc="f64")[0],
                                      f"largest rows T={T}")
            _log(f"  rel_l2={r[0]:.3e} max_abs={r[1]:.3e}")


def test_moe_zero_tokens(dev):
    torch, k3x = dev
    _log("case: moe T=0")
    E, H, I = 4, 128, 128
    pool = _pool(torch, k3x, S.device_pool(1, 0, E, H, I), E, H, I)
    ws = k3x.alloc_workspace(k3x.k3x_moe_workspace_size(pool, 0, 16))
    ws.fill_(0xFF)
    x = torch.empty((0, H), dtype=torch.int16, device="cuda")
    idx = torch.empty((0, 16), dtype=torch.int32, device="cuda")
    g = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    y = torch.empty((0, H), dtype=torch.float32, device="cuda")
    k3x.k3x_moe_forward(pool, x, 0, idx, g, 16, y, ws)
    assert k3x.k3x_fetch_drops(ws) == 0


def test_route_moe_zero_tokens_resets_the_drop_counter(dev):
    """An empty router + experts call leaves the workspace's drop counter at 0, as an empty
    k3x_moe_forward does, also after a call that dropped a slot on the same workspace."""
    torch, k3x = dev
    _log("case: route_moe T=0 after a call with a dropped slot")
    E, H, I, k = 8, 256, 256, 4
    pool = _pool(torch, k3x, S.device_pool(5, 0, E, H, I), E, H, I)
    W = S.normal_bf16(5, S.P_WR, 0, (E, H), std=0.05)
    r = k3x.router_desc(_t(torch, W), None, k, 1, 1.0)
    ws = k3x.alloc_workspace(max(k3x.k3x_route_moe_workspace_size(r, pool, 2),
                                 k3x.k3x_moe_workspace_size(pool, 2, k)))
    x = _t(torch, S.normal_bf16(5, S.P_X, 0, (2, H)))
    idx = torch.tensor([[0, 1, 2, E + 3], [4, 5, 6, 7]], dtype=torch.int32, device="cuda")
    g = torch.full((2, k), 0.25, dtype=torch.float32, device="cuda")
    y = torch.empty((2, H), dtype=torch.float32, device="cuda")
    k3x.k3x_moe_forward(pool, x, 2, idx, g, k, y, ws)
    assert k3x.k3x_fetch_drops(ws) == 1
    e0 = torch.empty((0,), dtype=torch.int32, device="cuda")
    k3x.k3x_route_moe_forward(r, pool, e0, 0, e0, e0, e0, ws)
    assert k3x.k3x_fetch_drops(ws) == 0


# ------------------------------------------------------------------------------------------
# router
# ------------------------------------------------------------------------------------------
def _route_both(torch, k3x, orc, x, W, b, topk, renorm=1, scale=1.0):
    idx, gates, _ = k3x.route_topk(_t(torch, W), None if b is None else _t(torch, b),
                                   _t(torch, x), topk, renorm, scale)
    torch.cuda.synchronize()
    i_ref, g_ref = orc.route(x, W, b, topk, renorm, scale)
    return _np(idx), _np(gates), i_ref, g_ref


def test_router_parity_k3_shape(dev, orc):
    torch, k3x = dev
    w = S.WORKLOADS[2]
    _log("case: router E=896 H=3584 T=96 topk=16")
    W, b = S.router_inputs(w)
    x = S.normal_bf16(4242, S.P_X, 0, (96, w.H))
    idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, 16)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))


def test_router_parity_zipf_bias(dev, orc):
    torch, k3x = dev
    w = S.WORKLOADS[3]
    _log("case: router Zipf bias T=64")
    W, b = S.router_inputs(w)
    x = S.normal_bf16(77, S.P_X, 0, (64, w.H))
    idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, 16)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))


def test_router_ties_full_k_and_options(dev, orc):
    torch, k3x = dev
    _log("case: router ties / k=E / renorm off / scale")
    E, H = 96, 256
    W = S.normal_bf16(3, S.P_WR, 0, (E, H), std=0.05)
    W[17] = W[4]
    b = S.normal_f32(3, S.P_BIAS, 0, (E,), std=0.01)
    b[4] = b[17] = 5.0
    x = S.normal_bf16(3, S.P_X, 0, (5, H))
    idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, 4)
    assert np.array_equal(idx, i_ref) and np.all(idx[:, 0] == 4) and np.all(idx[:, 1] == 17)
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))
    idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, E)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))
    idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, None, 8, renorm=0, scale=2.5)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))


def test_router_many_equal_scores(dev, orc):
    """Whole blocks of identical router rows and biases: selection falls back on the lower
    index among equal scores, including more equal scores than one LDS list holds."""
    torch, k3x = dev
    _log("case: router with 300 identical experts, E=700")
    E, H = 700, 128
    W = S.normal_bf16(11, S.P_WR, 0, (E, H), std=0.05)
    W[100:400] = W[100]
    b = S.normal_f32(11, S.P_BIAS, 0, (E,), std=0.01)
    b[100:400] = 3.0
    x = S.normal_bf16(11, S.P_X, 0, (3, H))
    for k in (16, 64, 333):
        idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, k)
        assert np.array_equal(idx, i_ref), k
        assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32)), k
    assert list(i_ref[0, :16]) == list(range(100, 116))


def test_router_selection_paths(dev, orc):
    """Selection at the boundaries of its register layouts (E up to 1024 and beyond, topk up
    to 64 and beyond; the sorting-network selection's limits E <= 1024, topk <= 16, with
    fewer experts than one quad's 16 words, one wave's 256 and the workgroup's 1024), ragged
    token counts, and biases that make +0 and -0 selection scores compare equal."""
    torch, k3x = dev
    for E, k, T in ((1024, 64, 7), (1024, 65, 3), (1025, 16, 5), (64, 64, 6), (2048, 16, 9),
                    (1024, 16, 4), (1, 1, 2), (5, 5, 3), (16, 16, 2), (17, 16, 2), (256, 16, 3),
                    (257, 1, 2), (300, 17, 2)):
        _log(f"case: router selection E={E} topk={k} T={T}")
        H = 256
        W = S.normal_bf16(E + k, S.P_WR, 0, (E, H), std=0.05)
        b = S.normal_f32(E + k, S.P_BIAS, 0, (E,), std=0.01)
        x = S.normal_bf16(E + k, S.P_X, 0, (T, H))
        idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, k)
        assert np.array_equal(idx, i_ref), (E, k, T)
        assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32)), (E, k, T)
    # zero router rows with zero bias next to equal ones with bias -0.0: score + bias is +0.5
    # or 0.5 + -0.0 = +0.5, so the keys tie and the lower index wins
    E, H = 128, 64
    W = S.normal_bf16(5, S.P_WR, 0, (E, H), std=0.05)
    W[10:20] = 0
    b = np.zeros(E, dtype=np.float32)
    b[10:15] = np.float32(-0.0)
    b[20:] = -1.0
    x = S.normal_bf16(5, S.P_X, 0, (4, H))
    idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, 8)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))


def test_router_shared_key_digits(dev, orc):
    """Selection scores that share their leading bytes: zero router rows give every expert
    the score 0.5 exactly, and biases that are multiples of its ulp (2^-24) or of 2^-16 make
    the keys differ only in their last byte, or only from the second byte down; with no bias
    every key is equal and the lowest indices are taken in order."""
    torch, k3x = dev
    E, H = 896, 512
    W = np.zeros((E, H), dtype=np.uint16)
    x = S.normal_bf16(3, S.P_X, 0, (2, H))
    rng = np.random.default_rng(3)
    cases = {
        "all equal": None,
        "last byte": (rng.integers(0, 256, E) * 2.0 ** -24).astype(np.float32),
        "two bytes": (rng.integers(0, 65536, E) * 2.0 ** -24).astype(np.float32),
    }
    for name, b in cases.items():
        _log(f"case: router keys sharing leading digits ({name})")
        for k in (16, 64):
            idx, gates, i_ref, g_ref = _route_both(torch, k3x, orc, x, W, b, k)
            assert np.array_equal(idx, i_ref), (name, k)
            assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32)), (name, k)
            if b is None:
                assert list(i_ref[0]) == list(range(k))


def _route_moe_both(torch, k3x, pool, Wd, bd, xd, T, k, renorm=1, scale=1.0):
    """k3x_route_moe_forward against k3x_route_topk + k3x_moe_forward on the same inputs."""
    r = k3x.router_desc(Wd, bd, k, renorm, scale)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, pool.H), dtype=torch.float32, device="cuda")
    ws = k3x.alloc_workspace(k3x.k3x_route_moe_workspace_size(r, pool, T))
    k3x.k3x_route_moe_forward(r, pool, xd, T, idx, gates, y, ws)
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    i2, g2, _ = k3x.route_topk(Wd, bd, xd, k, renorm, scale)
    y2, _ = k3x.moe_forward(pool, xd, i2, g2)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2) and torch.equal(gates.view(torch.int32), g2.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    return _np(idx), _np(gates), _np(y)


def test_route_moe_forward_equals_separate_calls(dev, orc):
    """Router and experts in one call: idx, gates and y equal the two separate calls bit for
    bit, and the oracle's router and forward; also more than 1024 experts (16 keys per
    selection thread), no bias, no renormalisation with a routed scale, SiTU-GLU, batches,
    and, for the single-token path that selects inside its W1/W3 launch, 64 picks of 1024
    and 300 tied selection scores."""
    torch, k3x = dev
    w = S.WORKLOADS[2]
    _log("case: route_moe one token, K3 shape")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    W, b = S.router_inputs(w)
    Wd, bd = _t(torch, W), _t(torch, b)
    cache = {}
    for t in range(3):
        x = S.normal_bf16(w.seed + 100 + t, S.P_X, 0, (1, w.H))
        idx, gates, y = _route_moe_both(torch, k3x, pool, Wd, bd, _t(torch, x), 1, w.topk)
        i_ref, g_ref = orc.route(x, W, b, w.topk)
        assert np.array_equal(idx, i_ref)
        assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))
        y_ref = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x, i_ref, g_ref, [0], cache=cache)
        assert np.array_equal(y, y_ref)
    _log("case: route_moe options (no bias; renorm 0 with routed scale 2.5; T = 5)")
    x = S.normal_bf16(w.seed + 200, S.P_X, 0, (5, w.H))
    _route_moe_both(torch, k3x, pool, Wd, None, _t(torch, x[:1]), 1, w.topk)
    _route_moe_both(torch, k3x, pool, Wd, bd, _t(torch, x[:1]), 1, w.topk, renorm=0, scale=2.5)
    _route_moe_both(torch, k3x, pool, Wd, bd, _t(torch, x), 5, w.topk)
    del pool
    _log("case: route_moe SiTU one token")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I, act=SITU)
    _route_moe_both(torch, k3x, pool, Wd, bd, _t(torch, x[:1]), 1, w.topk)
    del pool
    for E, H, I, k in ((2048, 512, 384, 16), (1025, 256, 256, 64), (64, 512, 512, 8),
                       (1024, 512, 256, 64), (700, 256, 256, 16), (700, 256, 256, 64)):
        _log(f"case: route_moe E={E} H={H} I={I} k={k}")
        pool = _pool(torch, k3x, S.device_pool(E, 0, E, H, I), E, H, I)
        W = S.normal_bf16(E, S.P_WR, 0, (E, H), std=0.05)
        b = S.normal_f32(E, S.P_BIAS, 0, (E,), std=0.01)
        if E == 700:  # 300 equal selection scores: ties go to the lower index
            W[100:400] = W[100]
            b[100:400] = 3.0
        x = S.normal_bf16(E, S.P_X, 0, (1, H))
        idx, gates, y = _route_moe_both(torch, k3x, pool, _t(torch, W), _t(torch, b),
                                        _t(torch, x), 1, k)
        i_ref, g_ref = orc.route(x, W, b, k)
        assert np.array_equal(idx, i_ref)
        assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32))
        del pool


def _residual_route_moe_both(torch, k3x, orc, pool, Wd, bd, x, y_prev, T, k, alias_y=False):
    """k3x_residual_route_moe_forward against k3x_residual_add_rmsnorm_bf16 (k3x_rmsnorm_bf16
    without y_prev) followed by k3x_route_moe_forward: x_next, xn, idx, gates and y equal bit
    for bit, x is left as it was, and x_next and xn equal the oracle's residual update and
    RMSNorm."""
    H = pool.H
    r = k3x.router_desc(Wd, bd, k)
    xd = _t(torch, x)
    yp = _t(torch, y_prev) if y_prev is not None else None
    x_next = torch.full_like(xd, 0x7F7F) if y_prev is not None else None
    xn = torch.full_like(xd, 0x7F7F)
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    gates = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    y = yp.clone() if alias_y else torch.full((T, H), float("nan"), device="cuda")
    ws = k3x.alloc_workspace(k3x.k3x_route_moe_workspace_size(r, pool, T))
    k3x.k3x_residual_route_moe_forward(r, pool, xd, y if alias_y else yp, 1e-6, x_next, xn, T,
                                       idx, gates, y, ws)
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    xr, xn2 = xd.clone(), torch.empty_like(xd)
    if y_prev is not None:
        k3x.k3x_residual_add_rmsnorm_bf16(xr, yp, T, H, 1e-6, xn2)
    else:
        k3x.k3x_rmsnorm_bf16(xd, T, H, 1e-6, xn2)
    idx2, gates2 = torch.empty_like(idx), torch.empty_like(gates)
    y2 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws2 = k3x.alloc_workspace(k3x.k3x_route_moe_workspace_size(r, pool, T))
    k3x.k3x_route_moe_forward(r, pool, xn2, T, idx2, gates2, y2, ws2)
    torch.cuda.synchronize()
    assert np.array_equal(_np(xd, np.uint16), x)
    x_ref = x if y_prev is None else orc.residual_add_bf16(x, y_prev)
    if y_prev is not None:
        assert torch.equal(x_next, xr)
        assert np.array_equal(_np(x_next, np.uint16), x_ref)
    assert torch.equal(xn, xn2)
    assert np.array_equal(_np(xn, np.uint16), orc.rmsnorm_bf16(x_ref, 1e-6))
    assert torch.equal(idx, idx2)
    assert torch.equal(gates.view(torch.int32), gates2.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def test_residual_route_moe_equals_separate_calls(dev, orc):
    """The residual update and RMSNorm in front of the router in one call: at one token the
    router's scores launch does both (K3 shape; 1022 experts of width 1024, whose last
    workgroup has idle waves); at several tokens or widths that are not multiples of 512 the
    separate norm launch runs first.  Also the first layer (no y_prev), y passed as y_prev, a
    contract pool, and the overlap checks."""
    torch, k3x = dev
    w = S.WORKLOADS[2]
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    W, b = S.router_inputs(w)
    Wd, bd = _t(torch, W), _t(torch, b)
    rng = np.random.default_rng(11)
    x = S.normal_bf16(w.seed + 300, S.P_X, 0, (3, w.H))
    yp = (rng.standard_normal((3, w.H)) * 0.5).astype(np.float32)
    for T, y_prev, alias in ((1, None, False), (1, yp[:1], False), (1, yp[:1], True),
                             (3, yp, False), (3, None, False)):
        _log(f"case: residual_route_moe K3 shape T={T} y_prev={y_prev is not None} "
             f"y_is_y_prev={alias}")
        _residual_route_moe_both(torch, k3x, orc, pool, Wd, bd, x[:T], y_prev, T, w.topk,
                                 alias_y=alias)
    _log("case: residual_route_moe overlap checks")
    r = k3x.router_desc(Wd, bd, w.topk)
    xd = _t(torch, x[:1])
    buf = torch.empty((4, w.H), dtype=torch.int16, device="cuda")
    ypd = _t(torch, yp[:1])
    idx = torch.empty((1, w.topk), dtype=torch.int32, device="cuda")
    gates = torch.empty((1, w.topk), dtype=torch.float32, device="cuda")
    y = torch.empty((1, w.H), dtype=torch.float32, device="cuda")
    ws = k3x.alloc_workspace(k3x.k3x_route_moe_workspace_size(r, pool, 1))
    for x_arg, x_next, xn in ((xd, xd, buf[0]), (xd, buf[0], buf[0]), (xd, buf[1], xd),
                              (buf[1], buf[0], buf[1])):
        with pytest.raises(k3x.K3xError) as err:
            k3x.k3x_residual_route_moe_forward(r, pool, x_arg, ypd, 1e-6, x_next, xn, 1, idx,
                                               gates, y, ws)
        assert err.value.status == k3x.K3X_E_INVALID_ARG
    with pytest.raises(k3x.K3xError) as err:  # xn inside y
        k3x.k3x_residual_route_moe_forward(r, pool, xd, ypd, 1e-6, buf[0], y, 1, idx, gates, y,
                                           ws)
    assert err.value.status == k3x.K3X_E_INVALID_ARG
    del pool
    for E, H, I, k, contract in ((1022, 1024, 256, 16, False), (64, 256, 256, 8, False),
                                 (64, 512, 512, 8, True)):
        _log(f"case: residual_route_moe E={E} H={H} I={I} k={k} contract={contract}")
        pool = k3x.k3x_expert_pool_create(S.device_pool(E, 0, E, H, I), hidden=H, inter=I,
                                          n_experts=E, contract=contract)
        W = S.normal_bf16(E, S.P_WR, 0, (E, H), std=0.05)
        b = S.normal_f32(E, S.P_BIAS, 0, (E,), std=0.01)
        x = S.normal_bf16(E + 1, S.P_X, 0, (2, H))
        yp = (rng.standard_normal((2, H)) * 0.5).astype(np.float32)
        for T in ((1,) if contract else (1, 2)):
            _residual_route_moe_both(torch, k3x, orc, pool, _t(torch, W), _t(torch, b), x[:T],
                                     yp[:T], T, k)
        del pool


# ------------------------------------------------------------------------------------------
# the five workloads at full size, every output checked
# ------------------------------------------------------------------------------------------
def test_workload1_decode_e64(dev, orc):
    torch, k3x = dev
    w = S.WORKLOADS[1]
    _log(f"case: workload {w.name}")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    x = S.activations(w)
    idx, gates = S.uniform_routing(w.seed, w.T, w.E, w.topk)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    y_ref = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x, idx, gates, range(w.T))
    r = assert_y_close(_np(y), y_ref, w.name)
    _log(f"  rel_l2={r[0]:.3e} max_abs={r[1]:.3e}")
    # single-token decode follows the oracle's arithmetic order: equal values
    assert np.array_equal(_np(y), y_ref), "single-token decode differs from the fp32 oracle"


def test_workload2_decode_e896_router(dev, orc):
    torch, k3x = dev
    w = S.WORKLOADS[2]
    _log(f"case: workload {w.name}")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    W, b = S.router_inputs(w)
    x = S.activations(w)
    xd = _t(torch, x)
    idx, gates, _ = k3x.route_topk(_t(torch, W), _t(torch, b), xd, w.topk)
    y, ws = k3x.moe_forward(pool, xd, idx, gates)
    torch.cuda.synchronize()
    i_ref, g_ref = orc.route(x, W, b, w.topk)
    assert np.array_equal(_np(idx), i_ref)
    assert np.array_equal(_np(gates).view(np.uint32), g_ref.view(np.uint32))
    y_ref = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x, i_ref, g_ref, range(w.T))
    r = assert_y_close(_np(y), y_ref, w.name)
    _log(f"  rel_l2={r[0]:.3e} max_abs={r[1]:.3e}")
    assert np.array_equal(_np(y), y_ref), "single-token decode differs from the fp32 oracle"
    del pool
    torch.cuda.empty_cache()


def test_decode_single_token_equals_oracle_many(dev, orc):
    """Single-token decode over 24 different tokens and routings of a 64-expert pool:
    every output equals the fp32 oracle's (same arithmetic order)."""
    torch, k3x = dev
    w = S.WORKLOADS[1]
    _log("case: single-token decode, 24 tokens, E=64, full shapes")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    x = S.normal_bf16(31337, S.P_X, 0, (24, w.H))
    idx, gates = S.uniform_routing(31337, 24, w.E, w.topk)
    cache = {}
    ws = None
    worst = 0.0
    for t in range(24):
        y, ws = k3x.moe_forward(pool, _t(torch, x[t:t + 1]), _t(torch, idx[t:t + 1]),
                                _t(torch, gates[t:t + 1]), ws=ws)
        torch.cuda.synchronize()
        y_ref = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x[t:t + 1], idx[t:t + 1],
                                       gates[t:t + 1], [0], cache=cache)
        worst = max(worst, y_errors(_np(y), y_ref)[0])
        assert np.array_equal(_np(y), y_ref), f"token {t}"
    _log(f"  worst rel_l2 over 24 tokens: {worst:.3e}")


def _whole_tensor_verdict(torch, orc, w, y, x, idx, gates, what, act="swiglu"):
    """The y verdict over the whole [T][H] output of a full-size run (every token), against
    the oracle walking the experts one by one; the fp64 oracle is computed only if the
    fallback needs it.  Logs the whole-tensor errors and the worst single token."""
    y_ref = oracle_forward_all(orc, w.seed, 0, w.H, w.I, x, idx, gates, act=act, log=_log)
    r = assert_y_close_oracle(
        y, y_ref, lambda: oracle_forward_all(orc, w.seed, 0, w.H, w.I, x, idx, gates, acc="f64",
                                             act=act, log=_log), what)
    rel, t_rel, mx, t_mx = token_errors(y, y_ref)
    _log(f"  {what}: whole tensor rel_l2={r[0]:.3e} max_abs={r[1]:.3e}; worst token rel_l2="
         f"{rel:.3e} (token {t_rel}), worst token max_abs={mx:.3e} (token {t_mx})")
    return r


def test_workload3_decode_t32_zipf(dev, orc):
    torch, k3x = dev
    w = S.WORKLOADS[3]
    _log(f"case: workload {w.name}")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    W, b = S.router_inputs(w)
    x = S.activations(w)
    xd = _t(torch, x)
    idx, gates, _ = k3x.route_topk(_t(torch, W), _t(torch, b), xd, w.topk)
    y, ws = k3x.moe_forward(pool, xd, idx, gates)
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    i_ref, g_ref = orc.route(x, W, b, w.topk)
    assert np.array_equal(_np(idx), i_ref)
    assert np.array_equal(_np(gates).view(np.uint32), g_ref.view(np.uint32))
    _log(f"  distinct experts U={len(np.unique(i_ref))}")
    yv = _np(y)
    del pool, ws, y
    torch.cuda.empty_cache()
    _whole_tensor_verdict(torch, orc, w, yv, x, i_ref, g_ref, w.name)


def test_workload4_prefill_t4096(dev, orc):
    torch, k3x = dev
    w = S.WORKLOADS[4]
    _log(f"case: workload {w.name}")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I)
    x = S.activations(w)
    idx, gates = S.uniform_routing(w.seed, w.T, w.E, w.topk)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    yv = _np(y)
    del pool, ws, y
    torch.cuda.empty_cache()
    _whole_tensor_verdict(torch, orc, w, yv, x, idx, gates, w.name)


# ------------------------------------------------------------------------------------------
# the format's edge cases on every path
# ------------------------------------------------------------------------------------------
EDGE_C0 = 5  # the x element that meets the scale-2 weights (kept at |x| = 1.5)


def _edge_pool(seed, E, H, I):
    """A host pool with the edge cases of the MXFP4 format (kimi-k3-in-c README, Part II
    section 4: the E2M1 table with its -0 code 8; the E8M0 scale 2^(s - 127), byte 255 zeroing
    its group), arranged so every output stays finite and of normal size:
      - NaN scale bytes (255) in about 4 % of the groups of W1, W3 and W2;
      - row 1 of every matrix all code 8 (-0), and about 5 % of the low nibbles set to 8;
      - scale byte 2: W3 rows 32..63 hold a single 6.0 (code 7) at element EDGE_C0 in a group
        of scale byte 2, so u = x[EDGE_C0] * 6 * 2^-125 there and h is up to about 1e-34 (a
        normal bf16); W2 row 7 has scale byte 2 in every group (a normal fp32 output near
        1e-31);
      - scale byte 252: W2 group 1 (the columns of those tiny h) has scale byte 252 in every
        row, which brings their products back to ordinary magnitudes (2^125 * 6 * 1e-34)."""
    pool = S.host_pool(seed, 0, E, H, I)
    rng = np.random.default_rng(seed)
    for name in ("w1", "w3", "w2"):
        p = pool[name + "_packed"]
        sc = pool[name + "_scale"]
        sc[rng.random(sc.shape) < 0.04] = 255
        p[:, 1, :] = 0x88
        m = rng.random(p.shape) < 0.05
        p[m] = (p[m] & 0xF0) | 0x08
    p3, s3 = pool["w3_packed"], pool["w3_scale"]
    p3[:, 32:64, :] = 0
    p3[:, 32:64, EDGE_C0 // 2] = 0x70 if EDGE_C0 % 2 else 0x07
    s3[:, 32:64, EDGE_C0 // 32] = 2
    s2 = pool["w2_scale"]
    s2[:, :, 1] = 252
    s2[:, 7, :] = 2
    return pool


@pytest.mark.parametrize("path,E,H,I,T,k", [("decode", 4, 512, 512, 1, 4),
                                            ("grouped", 4, 384, 256, 3, 3),
                                            ("prefill", 4, 512, 1024, 40, 2)])
def test_format_edge_cases(dev, orc, path, E, H, I, T, k):
    """Scale byte 255, code 8 (-0) and the extreme scale bytes 2 and 252 reach the kernels of
    each path: the exact single-token decode equals the fp32 oracle bit for bit; the grouped
    and sorted-tile paths meet the y verdict, and so does output element 7 (W2's all-scale-2
    row) on its own."""
    torch, k3x = dev
    _log(f"case: format edge cases, {path} path E={E} H={H} I={I} T={T} k={k}")
    seed = 4000 + H + I + T
    host = _edge_pool(seed, E, H, I)
    devp = {n: _t(torch, host[n]) for n in S.TENSOR_NAMES}
    pool = _pool(torch, k3x, devp, E, H, I)
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    x[:, EDGE_C0] = np.where(np.arange(T) % 2 == 0, 0x3FC0, 0xBFC0)  # +-1.5
    x[0, 9] = 0x8000  # -0
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, gates = S.uniform_routing(seed, T, k, k)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    yv = _np(y)
    y_ref, drops = orc.moe_forward(host, x, idx, gates)
    assert drops == 0 and np.all(np.isfinite(y_ref))
    # the tiny h rows really reach W2 through the scale-252 group: without them y changes
    flat = {n: a.copy() for n, a in host.items()}
    flat["w2_scale"][:, :, 1] = 255
    y_wo, _ = orc.moe_forward(flat, x, idx, gates)
    assert y_errors(y_wo, y_ref)[0] > 1e-3
    col = np.abs(y_ref[:, 7])
    assert np.all(col < 1e-25) and np.all(col[col > 0] > 1e-37)
    assert np.all(np.isfinite(yv)), "non-finite output"
    if path == "decode":
        assert np.array_equal(yv, y_ref), "single-token decode differs from the fp32 oracle"
        return
    r = assert_y_close_oracle(yv, y_ref, lambda: orc.moe_forward(host, x, idx, gates, acc="f64")[0],
                              f"edge {path}")
    rc = assert_y_close(yv[:, 7:8], y_ref[:, 7:8], f"edge {path}, the all-scale-2 row")
    _log(f"  rel_l2={r[0]:.3e} max_abs={r[1]:.3e}; scale-2 row rel_l2={rc[0]:.3e}")


# ------------------------------------------------------------------------------------------
# SiTU-GLU (the engine's own activation) on every path
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("caps", [(4.0, 25.0), (0.5, 3.0)])
def test_situ_decode_bit_exact(dev, orc, caps):
    """Single-token decode with SiTU-GLU at full shapes (E = 64, 16 slots) and with small
    caps that saturate often: y equals the fp32 oracle bit for bit."""
    torch, k3x = dev
    w = S.WORKLOADS[1]
    act = ("situ",) + caps
    _log(f"case: SiTU decode caps={caps}")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I, act)
    x = S.normal_bf16(w.seed + 3, S.P_X, 0, (1, w.H))
    idx, gates = S.uniform_routing(w.seed + 3, 1, w.E, w.topk)
    y, _ = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    y_ref = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x, idx, gates, [0], act=act)
    assert np.array_equal(_np(y), y_ref)
    y_sw = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x, idx, gates, [0])
    assert not np.allclose(y_ref, y_sw)


@pytest.mark.parametrize("E,H,I,T,k", [(5, 256, 384, 8, 3), (4, 512, 512, 40, 2),
                                       (16, 1024, 512, 2, 8)])
def test_situ_grouped_and_prefill_paths(dev, orc, E, H, I, T, k):
    """Batches with SiTU-GLU on the small-batch grouped kernels (H = 256) and on the
    sorted-tile kernels (H = 512, 1024), against the oracle with the same activation."""
    torch, k3x = dev
    _log(f"case: SiTU E={E} H={H} I={I} T={T} k={k}")
    seed = 3000 + E + H + I + T
    host = S.host_pool(seed, 0, E, H, I)
    pool = _pool(torch, k3x, S.device_pool(seed, 0, E, H, I), E, H, I, SITU)
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    _, gates = S.uniform_routing(seed, T, k, k)
    y, _ = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    y_ref, _ = orc.moe_forward(host, x, idx, gates, act=SITU)
    r = assert_y_close_oracle(
        _np(y), y_ref, lambda: orc.moe_forward(host, x, idx, gates, acc="f64", act=SITU)[0],
        f"SiTU E={E} H={H} I={I} T={T} k={k}")
    _log(f"  rel_l2={r[0]:.3e} max_abs={r[1]:.3e}")


def test_situ_workload2_and_prefill_full_size(dev, orc):
    """Full shapes with SiTU-GLU: one routed decode token over 896 experts (bit-exact) and
    the 4096-token prefill (every token, tolerance)."""
    torch, k3x = dev
    w = S.WORKLOADS[2]
    _log("case: SiTU workload decode_t1_e896_router")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I, SITU)
    W, b = S.router_inputs(w)
    x = S.activations(w)
    xd = _t(torch, x)
    idx, gates, _ = k3x.route_topk(_t(torch, W), _t(torch, b), xd, w.topk)
    y, _ = k3x.moe_forward(pool, xd, idx, gates)
    torch.cuda.synchronize()
    y_ref = oracle_forward_sampled(orc, w.seed, 0, w.H, w.I, x, _np(idx), _np(gates), [0],
                                   act=SITU)
    assert np.array_equal(_np(y), y_ref)
    del pool
    w = S.WORKLOADS[4]
    _log("case: SiTU workload prefill_t4096_e896")
    pool = _pool(torch, k3x, S.device_pool(w.seed, 0, w.E, w.H, w.I), w.E, w.H, w.I, SITU)
    x = S.activations(w)
    idx, gates = S.uniform_routing(w.seed, w.T, w.E, w.topk)
    y, ws = k3x.moe_forward(pool, _t(torch, x), _t(torch, idx), _t(torch, gates))
    torch.cuda.synchronize()
    yv = _np(y)
    del pool, ws, y
    torch.cuda.empty_cache()
    _whole_tensor_verdict(torch, orc, w, yv, x, idx, gates, "SiTU prefill", act=SITU)


# ------------------------------------------------------------------------------------------
# RMSNorm / residual and a chained decode (teacher-forced per layer)
# ------------------------------------------------------------------------------------------
def test_rmsnorm_and_residual_bitwise(dev, orc):
    torch, k3x = dev
    _log("case: rmsnorm / residual T=33 H=3584")
    T, H = 33, 3584
    x = S.normal_bf16(8, S.P_X, 0, (T, H))
    xd = _t(torch, x)
    out = torch.empty_like(xd)
    k3x.k3x_rmsnorm_bf16(xd, T, H, 1e-6, out)
    y = np.random.default_rng(8).standard_normal((T, H)).astype(np.float32) * 30
    yd = _t(torch, y)
    xr = xd.clone()
    k3x.k3x_residual_add_bf16(xr, yd, T, H)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out, np.uint16), orc.rmsnorm_bf16(x, 1e-6))
    assert np.array_equal(_np(xr, np.uint16), orc.residual_add_bf16(x, y))
    # the fused residual + RMSNorm: both outputs equal the oracle's two steps bit for bit
    for H2 in (H, 8200):  # 8200 > 64 * 8 * 8 takes the wide variant
        x2 = S.normal_bf16(9, S.P_X, 0, (T, H2))
        y2 = np.random.default_rng(9).standard_normal((T, H2)).astype(np.float32) * 30
        xf, yf = _t(torch, x2), _t(torch, y2)
        nf = torch.empty_like(xf)
        k3x.k3x_residual_add_rmsnorm_bf16(xf, yf, T, H2, 1e-6, nf)
        torch.cuda.synchronize()
        x_ref = orc.residual_add_bf16(x2, y2)
        assert np.array_equal(_np(xf, np.uint16), x_ref), H2
        assert np.array_equal(_np(nf, np.uint16), orc.rmsnorm_bf16(x_ref, 1e-6)), H2


def _chain(torch, k3x, orc, L, E, log_every=True):
    w = S.WORKLOADS[5]
    H, I, k = w.H, w.I, w.topk
    x = S.activations(w)
    xd = _t(torch, x)
    worst = 0.0
    # layer l's residual update and layer l + 1's RMSNorm run as one fused launch
    xn = torch.empty_like(xd)
    k3x.k3x_rmsnorm_bf16(xd, 1, H, 1e-6, xn)
    for layer in range(L):
        pool = _pool(torch, k3x, S.device_pool(w.seed, layer, E, H, I), E, H, I)
        W = S.normal_bf16(w.seed, S.P_WR, layer, (E, H), std=0.02)
        b = S.zipf_bias(w.seed, E, layer)
        x_in = _np(xd, np.uint16).copy()
        idx, gates, _ = k3x.route_topk(_t(torch, W), _t(torch, b), xn, k)
        y, _ = k3x.moe_forward(pool, xn, idx, gates)
        if layer + 1 < L:
            xn_next = torch.empty_like(xd)
            k3x.k3x_residual_add_rmsnorm_bf16(xd, y, 1, H, 1e-6, xn_next)
        else:
            k3x.k3x_residual_add_bf16(xd, y, 1, H)
        torch.cuda.synchronize()
        # teacher forcing: the oracle takes this layer's GPU input
        xn_ref = orc.rmsnorm_bf16(x_in, 1e-6)
        assert np.array_equal(_np(xn, np.uint16), xn_ref), layer
        i_ref, g_ref = orc.route(xn_ref, W, b, k)
        assert np.array_equal(_np(idx), i_ref), layer
        assert np.array_equal(_np(gates).view(np.uint32), g_ref.view(np.uint32)), layer
        y_ref = oracle_forward_sampled(orc, w.seed, layer, H, I, xn_ref, i_ref, g_ref, [0])
        rel, mx = assert_y_close(_np(y), y_ref, f"layer {layer}")
        assert np.array_equal(_np(y), y_ref), f"layer {layer}: differs from the fp32 oracle"
        assert np.array_equal(_np(xd, np.uint16), orc.residual_add_bf16(x_in, y_ref)), layer
        if layer + 1 < L:
            xn = xn_next
        worst = max(worst, rel)
        if log_every:
            _log(f"  layer {layer}: rel_l2={rel:.3e} max_abs={mx:.3e}")
        del pool
    return worst


def _chain_fused(torch, k3x, orc, L, E, log_every=True):
    """The chain as the benchmark runs it: one k3x_residual_route_moe_forward per layer (the
    previous layer's residual update, this layer's RMSNorm, router and experts), two x
    buffers taking turns, one y buffer that is both y_prev and y, and a last residual add."""
    w = S.WORKLOADS[5]
    H, I, k = w.H, w.I, w.topk
    x = S.activations(w)
    bufs = [_t(torch, x), torch.empty((1, H), dtype=torch.int16, device="cuda"),
            torch.empty((1, H), dtype=torch.int16, device="cuda")]
    x_cur = bufs[0]
    xn = torch.empty_like(x_cur)
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((1, k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
    worst, ws = 0.0, None
    for layer in range(L):
        pool = _pool(torch, k3x, S.device_pool(w.seed, layer, E, H, I), E, H, I)
        W = S.normal_bf16(w.seed, S.P_WR, layer, (E, H), std=0.02)
        b = S.zipf_bias(w.seed, E, layer)
        r = k3x.router_desc(_t(torch, W), _t(torch, b), k)
        if ws is None:
            ws = k3x.alloc_workspace(k3x.k3x_route_moe_workspace_size(r, pool, 1))
        x_in = _np(x_cur, np.uint16).copy()
        y_in = _np(y).copy() if layer else None
        x_next = bufs[1] if x_cur is not bufs[1] else bufs[2]
        k3x.k3x_residual_route_moe_forward(r, pool, x_cur, y if layer else None, 1e-6,
                                           x_next if layer else None, xn, 1, idx, gates, y, ws)
        torch.cuda.synchronize()
        assert k3x.k3x_fetch_drops(ws) == 0
        # teacher forcing: the oracle takes this layer's GPU inputs
        x_ref = orc.residual_add_bf16(x_in, y_in) if layer else x_in
        if layer:
            assert np.array_equal(_np(x_next, np.uint16), x_ref), layer
            x_cur = x_next
        xn_ref = orc.rmsnorm_bf16(x_ref, 1e-6)
        assert np.array_equal(_np(xn, np.uint16), xn_ref), layer
        i_ref, g_ref = orc.route(xn_ref, W, b, k)
        assert np.array_equal(_np(idx), i_ref), layer
        assert np.array_equal(_np(gates).view(np.uint32), g_ref.view(np.uint32)), layer
        y_ref = oracle_forward_sampled(orc, w.seed, layer, H, I, xn_ref, i_ref, g_ref, [0])
        rel, mx = assert_y_close(_np(y), y_ref, f"layer {layer}")
        assert np.array_equal(_np(y), y_ref), f"layer {layer}: differs from the fp32 oracle"
        worst = max(worst, rel)
        if log_every:
            _log(f"  layer {layer}: rel_l2={rel:.3e} max_abs={mx:.3e}")
        del pool
    x_in = _np(x_cur, np.uint16).copy()
    k3x.k3x_residual_add_bf16(x_cur, y, 1, H)
    torch.cuda.synchronize()
    assert np.array_equal(_np(x_cur, np.uint16), orc.residual_add_bf16(x_in, _np(y)))
    return worst


def test_chain12_reduced_pool(dev, orc):
    """Twelve chained layers (RMSNorm -> router -> experts -> residual) with 64 experts per
    layer, as separate calls and as one fused call per layer; every layer is checked against
    the oracle on the GPU's own layer input."""
    torch, k3x = dev
    _log("case: chain of 12 layers, E=64, separate calls")
    _chain(torch, k3x, orc, 12, 64)
    _log("case: chain of 12 layers, E=64, fused calls")
    _chain_fused(torch, k3x, orc, 12, 64)


def test_chain12_full_size(dev, orc):
    """The chained workload at its full size, run as the benchmark runs it: 12 layers of 896
    experts with per-layer router weights and Zipf-skewed bias, one fused residual + RMSNorm
    + router + experts call per layer.  Layers are generated one after another (one 15.7 GB
    pool on the device at a time); each is checked against the oracle on the GPU's own input:
    residual update and RMSNorm bitwise, routing bit-exact, y equal to the fp32 oracle bit
    for bit."""
    torch, k3x = dev
    _log("case: chain of 12 layers, E=896 (full size), fused calls")
    _chain_fused(torch, k3x, orc, 12, 896)
