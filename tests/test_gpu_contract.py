"""GPU parity of the floating point contract's arithmetic (a pool created with contract = 1):
one token's expert forward equals the oracle's contract forward (oracle_expert_forward_contract
+ the fp32 slot-order combine) bit for bit."""
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


def _contract_ref(orc, seed, layer, H, I, x_bits, idx, gates, E, act):
    k = idx.shape[1]
    d = np.zeros((1, k, H), dtype=np.float32)
    valid = np.zeros((1, k), dtype=np.uint8)
    for j in range(k):
        e = int(idx[0, j])
        if 0 <= e < E:
            d[0, j] = orc.expert_forward_contract(x_bits[0], S.expert_bytes(seed, layer, e, H, I), act=act)
            valid[0, j] = 1
    return orc.combine(gates, d, valid)


def _run(torch, k3x, orc, seed, E, H, I, k, act="swiglu", drop=False):
    kw = {} if act == "swiglu" else {"activation": "situ", "situ_b1": act[1], "situ_b2": act[2]}
    pool = k3x.k3x_expert_pool_create(S.device_pool(seed, 0, E, H, I), hidden=H, inter=I,
                                      n_experts=E, contract=True, **kw)
    x = S.normal_bf16(seed, S.P_X, 0, (1, H))
    idx, gates = S.uniform_routing(seed, 1, E, k)
    if drop:
        idx[0, 1] = E + 3
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    y, ws = k3x.moe_forward(pool, xd, torch.from_numpy(idx).cuda(), torch.from_numpy(gates).cuda())
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == (1 if drop else 0)
    y_ref = _contract_ref(orc, seed, 0, H, I, x, idx, gates, E, act)
    got = y.cpu().numpy()
    bad = int((got != y_ref).sum())
    assert bad == 0, f"E={E} H={H} I={I} k={k} act={act}: {bad} of {got.size} differ, " \
        f"rel {np.linalg.norm(got - y_ref) / np.linalg.norm(y_ref):.2e}"
    return got


@pytest.mark.parametrize("E,H,I,k", [(8, 256, 384, 3), (6, 512, 128, 5), (20, 1024, 768, 16)])
def test_contract_small(dev, orc, E, H, I, k):
    torch, k3x = dev
    _log(f"case: contract E={E} H={H} I={I} k={k}")
    _run(torch, k3x, orc, 300 + H + k, E, H, I, k)


def test_contract_situ_drop_and_largest_rows(dev, orc):
    torch, k3x = dev
    _log("case: contract SiTU-GLU with a dropped slot")
    _run(torch, k3x, orc, 411, 10, 512, 384, 6, act=("situ", 4.0, 25.0), drop=True)
    _log("case: contract rows of 128 groups (H = I = 4096)")
    _run(torch, k3x, orc, 412, 4, 4096, 4096, 2)


def test_contract_k3_shape(dev, orc):
    """The K3 expert shape with the router's own pick of 16 of 896 experts; the contract
    result differs from the routed path's arithmetic (h in bf16) as expected."""
    torch, k3x = dev
    w = S.WORKLOADS[2]
    _log("case: contract at the K3 shape, 16 of 896 experts")
    got = _run(torch, k3x, orc, w.seed, w.E, w.H, w.I, w.topk)
    pool = k3x.k3x_expert_pool_create(S.device_pool(w.seed, 0, w.E, w.H, w.I), hidden=w.H,
                                      inter=w.I, n_experts=w.E)
    x = S.normal_bf16(w.seed, S.P_X, 0, (1, w.H))
    idx, gates = S.uniform_routing(w.seed, 1, w.E, w.topk)
    y, _ = k3x.moe_forward(pool, torch.from_numpy(x.view(np.int16)).cuda(),
                           torch.from_numpy(idx).cuda(), torch.from_numpy(gates).cuda())
    torch.cuda.synchronize()
    rel = float(np.linalg.norm(y.cpu().numpy() - got) / np.linalg.norm(got))
    _log(f"  routed path vs contract: rel {rel:.2e}")
    assert 0 < rel < 1e-2


def test_contract_empty_call_resets_the_drop_counter(dev, orc):
    """T = 0 on a contract pool enqueues only the reset of the workspace's drop counter."""
    torch, k3x = dev
    E, H, I, k = 6, 256, 384, 3
    _log("case: contract T = 0 after a call with a dropped slot")
    pool = k3x.k3x_expert_pool_create(S.device_pool(7, 0, E, H, I), hidden=H, inter=I,
                                      n_experts=E, contract=True)
    x = torch.from_numpy(S.normal_bf16(7, S.P_X, 0, (1, H)).view(np.int16)).cuda()
    idx = torch.tensor([[0, E + 1, 2]], dtype=torch.int32, device="cuda")
    gates = torch.full((1, k), 1.0 / k, dtype=torch.float32, device="cuda")
    y, ws = k3x.moe_forward(pool, x, idx, gates)
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 1
    y0 = y.clone()
    k3x.k3x_moe_forward(pool, x, 0, idx, gates, k, y, ws)
    torch.cuda.synchronize()
    assert k3x.k3x_fetch_drops(ws) == 0
    assert torch.equal(y, y0)  # nothing else was written
