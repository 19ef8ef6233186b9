"""GPU parity of the latent MoE block (router on the full width, bf16 down-projection, the
routed experts on the latent, RMSNorm of their aggregate, up-projection, the shared experts
added unweighted) through the C ABI, against the oracle.

Every dense product of the block is the contract's bf16 matmul in a fixed order on both
sides, so the checks are stage by stage, each against the oracle:
  - routing (idx, gates), the latent z and the shared activation s: bit for bit, from x alone;
  - the aggregate of the routed experts: against the oracle's routed forward on that z, with
    the verdict of the routed path (bit for bit on one token, whose decode kernels keep the
    oracle's order; relative L2 <= 1e-4 and max-abs <= 1e-3 of max|acc| on batches, whose
    sorted-tile kernels sum in another order);
  - the output: bit for bit against the oracle's tail (RMSNorm of the aggregate, up, sh2, the
    fp32 add) on the GPU's aggregate;
  - on one token the whole block bit for bit against the oracle's latent block.
On batches the end-to-end output is not held to a tolerance of its own: one bf16 rounding of
the normalised aggregate that falls the other way (its input differing in the last bits) moves
a token's output by about 2^-8 / sqrt(L) relative, more than the routed path's tolerance at
small L.  Inputs are seeded (k3x_synth); expected values come from the oracle only.
"""
import sys

import numpy as np
import pytest

import k3x_synth as S
from cases import assert_y_close_oracle

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


def _np(t):
    return t.detach().cpu().numpy()


def _act_name(act):
    return act if isinstance(act, str) else act[0]


def _host_pool_for(seed, layer, E, H, I, experts):
    """Host copies of the pool with only the listed experts filled in; the others stay
    untouched zero pages (the oracle reads only the experts it routes to)."""
    out = {}
    for t, n in enumerate(S.TENSOR_NAMES):
        rows, cols = S.tensor_shape(t, H, I)
        out[n] = np.zeros((E, rows, cols), dtype=np.uint8)
    for e in sorted(set(int(v) for v in experts)):
        ex = S.expert_bytes(seed, layer, e, H, I)
        for n in S.TENSOR_NAMES:
            out[n][e] = getattr(ex, n)
    return out


def _run(torch, k3x, orc, seed, T, D, L, I, n_shared, E, k, act, act_shared, norm=True,
         unit_weight=False, full_host=True):
    Sx = n_shared * I
    w = S.latent_inputs(seed, 0, D, L, Sx, E)
    x = S.normal_bf16(seed, S.P_X, 0, (T, D))
    b1, b2 = (4.0, 25.0) if _act_name(act) == "swiglu" else act[1:]
    sb1, sb2 = (4.0, 25.0) if _act_name(act_shared) == "swiglu" else act_shared[1:]
    pool = k3x.k3x_expert_pool_create(S.device_pool(seed, 0, E, L, I), hidden=L, inter=I,
                                      n_experts=E, activation=_act_name(act), situ_b1=b1,
                                      situ_b2=b2)
    dv = {n: _t(torch, w[n]) for n in ("Wr", "bias", "down", "up", "sh1", "sh3", "sh2", "norm_w")}
    norm_w = None if (unit_weight or not norm) else dv["norm_w"]
    d = k3x.latent_desc(dv["down"], dv["up"], dv["sh1"], dv["sh3"], dv["sh2"], norm_w, eps=1e-6,
                        latent_norm=int(norm), shared_activation=_act_name(act_shared),
                        situ_b1=sb1, situ_b2=sb2)
    r = k3x.router_desc(dv["Wr"], dv["bias"], k)
    xd = _t(torch, x)
    out = torch.empty((T, D), dtype=torch.float32, device="cuda")
    need = k3x.k3x_latent_workspace_size(d, pool, r, T)
    assert need > 0, k3x.k3x_last_error()
    ws = k3x.alloc_workspace(need)
    k3x.k3x_latent_forward(d, pool, r, xd, T, out, ws)
    torch.cuda.synchronize()
    lay = k3x.k3x_latent_ws_layout(d, pool, r, T)
    assert k3x.k3x_fetch_drops(ws[lay["moe"]:]) == 0
    got = _np(out)
    B = _np(ws)
    view = lambda name, dt, n: B[lay[name]:lay[name] + n * np.dtype(dt).itemsize].view(dt)
    idx = view("idx", np.int32, T * k).reshape(T, k)
    gates = view("gates", np.float32, T * k).reshape(T, k)
    z = view("z", np.uint16, T * L).reshape(T, L)
    acc = view("acc", np.float32, T * L).reshape(T, L)
    s_ = view("s", np.uint16, T * Sx).reshape(T, Sx)
    what = f"latent T={T} D={D} L={L} I={I} E={E} k={k}"

    # routing, z and s from x alone
    i_ref, g_ref = orc.route(x, w["Wr"], w["bias"], k)
    assert np.array_equal(idx, i_ref), what
    assert np.array_equal(gates.view(np.uint32), g_ref.view(np.uint32)), what
    z_ref = np.stack([orc.bf16_round(orc.dense64_bf16(w["down"], x[t])) for t in range(T)])
    assert np.array_equal(z, z_ref), f"{what}: z differs in {int((z != z_ref).sum())} places"
    g = np.stack([orc.dense64_bf16(w["sh1"], x[t]) for t in range(T)])
    u = np.stack([orc.dense64_bf16(w["sh3"], x[t]) for t in range(T)])
    s_ref = orc.bf16_round(orc.glu(g, u, act_shared))
    assert np.array_equal(s_, s_ref), f"{what}: s differs in {int((s_ != s_ref).sum())} places"

    # the routed experts on z
    if full_host:
        host = S.host_pool(seed, 0, E, L, I)
    else:
        host = _host_pool_for(seed, 0, E, L, I, i_ref.ravel())
    acc_ref, drops = orc.moe_forward(host, z_ref, i_ref, g_ref, act=act)
    assert drops == 0
    if T == 1:
        assert np.array_equal(acc, acc_ref), f"{what}: aggregate differs from the fp32 oracle"
    else:
        r = assert_y_close_oracle(
            acc, acc_ref, lambda: orc.moe_forward(host, z_ref, i_ref, g_ref, acc="f64", act=act)[0],
            f"{what}: aggregate")
        _log(f"  aggregate rel_l2={r[0]:.3e} max_abs={r[1]:.3e}")

    # the tail on the GPU's aggregate
    if not norm:
        nw = None
    elif unit_weight:
        nw = np.ones(L, dtype=np.float32)
    else:
        nw = w["norm_w"]
    a_t = orc.rmsnorm_w_f32(acc, nw, 1e-6) if norm else orc.bf16_round(acc)
    tail = np.stack([orc.dense64_bf16(w["up"], a_t[t]) + orc.dense64_bf16(w["sh2"], s_ref[t])
                     for t in range(T)]).astype(np.float32)
    assert np.array_equal(got, tail), f"{what}: output differs from the oracle's tail " \
        f"in {int((got != tail).sum())} places"

    # the whole block
    full, drops = orc.latent_block(x, w["Wr"], w["bias"], k, w["down"], w["up"], w["sh1"],
                                   w["sh3"], w["sh2"], nw, 1e-6, host, act=act,
                                   act_shared=act_shared)
    assert drops == 0
    rel = float(np.linalg.norm(got - full) / np.linalg.norm(full))
    _log(f"  end to end rel_l2={rel:.3e}")
    if T == 1:
        assert np.array_equal(got, full), f"{what}: block differs from the fp32 oracle"
    return got


SITU = ("situ", 4.0, 25.0)


@pytest.mark.parametrize("T", [1, 3, 9, 17])
def test_latent_block_small(dev, orc, T):
    """Several rows per wave, both token templates (1 and 8 per launch), passes of 8 tokens
    with a ragged last one, the routed experts on both decode and sorted-tile paths."""
    torch, k3x = dev
    _log(f"case: latent block small T={T}")
    _run(torch, k3x, orc, 500 + T, T, 1024, 512, 256, 2, 8, 2, "swiglu", SITU)


@pytest.mark.parametrize("norm,unit,act_shared", [(False, False, "swiglu"), (True, True, SITU),
                                                  (True, False, "swiglu")])
def test_latent_block_norm_and_activation_options(dev, orc, norm, unit, act_shared):
    """Without the latent norm (a = bf16 of the aggregate), the norm with weight 1, and
    SwiGLU shared experts; odd chunk counts per lane (D = 1536, L + S = 1536)."""
    torch, k3x = dev
    _log(f"case: latent block options norm={norm} unit_weight={unit} shared={act_shared}")
    for T in (1, 5):
        _run(torch, k3x, orc, 600 + T + 10 * norm + 20 * unit, T, 1536, 512, 512, 2, 6, 3,
             SITU, act_shared, norm=norm, unit_weight=unit)


def test_latent_block_many_experts(dev, orc):
    """Many experts, k above half of them: the router's ties and renormalisation on the full
    width, the sorted-tile path with most experts active."""
    torch, k3x = dev
    _log("case: latent block E=32 k=20 T=6")
    _run(torch, k3x, orc, 700, 6, 2048, 1024, 512, 2, 32, 20, "swiglu", SITU)


@pytest.mark.parametrize("T", [1, 8])
def test_latent_block_k3_full_size(dev, orc, T):
    """The K3 block at its full size: D 7168, latent 3584, 896 experts of 3072, top-16, two
    shared experts of 3072 (S 6144), SiTU-GLU shared experts, SwiGLU routed experts."""
    torch, k3x = dev
    sh = S.LATENT_K3
    _log(f"case: latent block K3 full size T={T}")
    _run(torch, k3x, orc, S.LATENT_SEED, T, sh.D, sh.L, sh.I, sh.n_shared, sh.E, sh.topk,
         "swiglu", SITU, full_host=False)
