"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a value printed on the
pages (tests/golden/), a hand-worked example, a closed form, an invariant, or brute force
through numpy's float64 dense algebra on tiny shapes.
"""
import json
import math
import os

import numpy as np
import pytest

import k3x_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------
# independent decoders written in the test (closed forms from the bit layout)
# ------------------------------------------------------------------------------------------
def e2m1_closed(code):
    """E2M1 from its bits: sign b3, exponent b2b1 (bias 1), mantissa b0; e = 0 is subnormal."""
    sgn = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sgn * mag


E2M1_NP = np.array([e2m1_closed(c) for c in range(16)], dtype=np.float64)


def dequant64(packed, scales):
    """Dense float64 matrix of an MXFP4 tensor: low nibble is the even column."""
    rows, half = packed.shape
    K = 2 * half
    codes = np.empty((rows, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    w = E2M1_NP[codes]
    sc = np.where(scales == 255, 0.0, np.ldexp(1.0, scales.astype(np.int64) - 127))
    return w * np.repeat(sc, 32, axis=1)


def bf16_rne_from64(v):
    """Round float64 values to bf16 (RNE) exactly, returning float64 values."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    for i, a in enumerate(v.ravel()):
        if a == 0.0:
            out.ravel()[i] = a
            continue
        e = math.frexp(a)[1]  # a = m * 2^e, 0.5 <= |m| < 1
        ulp = 2.0 ** (e - 8)  # bf16 keeps 8 significant bits
        q = a / ulp
        fl = math.floor(q)
        rem = q - fl
        if rem > 0.5 or (rem == 0.5 and fl % 2 == 1):
            fl += 1
        out.ravel()[i] = fl * ulp
    return out


def bits_to_f(b):
    return S.bf16_bits_to_f32(b).astype(np.float64)


# ------------------------------------------------------------------------------------------
# tables
# ------------------------------------------------------------------------------------------
def test_e2m1_table_matches_page(orc):
    g = _golden("e2m1_lut.json")
    lut = g["e2m1_lut"]
    assert len(lut) == 16
    for code, v in enumerate(lut):
        got = orc.e2m1(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), code


def test_e2m1_closed_form(orc):
    for code in range(16):
        v = e2m1_closed(code)
        got = orc.e2m1(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v)


def test_e8m0_powers_and_nan_byte(orc):
    for s in range(255):
        assert orc.e8m0(s) == math.ldexp(1.0, s - 127)
    assert orc.e8m0(255) == 0.0


def test_expert_layout_bytes():
    g = _golden("expert_layout.json")
    H, I = g["hidden"], g["inter"]
    assert S.expert_bytes_per_expert(H, I) == g["bytes_per_expert"]
    assert g["params_per_expert"] * 17 // 32 == g["bytes_per_expert"]  # 0.53125 B per weight
    names = {S.W1_PACKED: "w1_packed", S.W1_SCALE: "w1_scale", S.W3_PACKED: "w3_packed",
             S.W3_SCALE: "w3_scale", S.W2_PACKED: "w2_packed", S.W2_SCALE: "w2_scale"}
    for t, n in names.items():
        shp = S.tensor_shape(t, H, I)
        assert list(shp) == g["tensors"][n]["shape"]
        assert shp[0] * shp[1] == g["tensors"][n]["bytes"]


def test_bf16_helpers(orc):
    # widening is a 16-bit shift; rounding is RNE including ties to even
    assert orc.bf16_to_f32(0x3F80) == 1.0
    assert orc.bf16_to_f32(0xC0C0) == -6.0
    assert orc.f32_to_bf16(1.0) == 0x3F80
    tie_down = np.array([0x3F808000], dtype=np.uint32).view(np.float32)[0]  # 1 + 2^-8: tie, even is 1.0
    tie_up = np.array([0x3F818000], dtype=np.uint32).view(np.float32)[0]    # tie, rounds up to even
    assert orc.f32_to_bf16(float(tie_down)) == 0x3F80
    assert orc.f32_to_bf16(float(tie_up)) == 0x3F82
    rng = np.random.default_rng(0)
    v = rng.standard_normal(2000).astype(np.float32) * 100
    want = bf16_rne_from64(v.astype(np.float64))
    got = np.array([orc.bf16_to_f32(orc.f32_to_bf16(float(a))) for a in v])
    assert np.array_equal(got, want)
    # the array form: the same roundings, the ties, infinities and a NaN that stays a NaN
    vv = np.concatenate([v, np.array([tie_down, tie_up, np.inf, -np.inf], dtype=np.float32)])
    bits = orc.bf16_round(vv)
    assert np.array_equal(bits_to_f(bits[:2000]), want)
    assert list(bits[2000:]) == [0x3F80, 0x3F82, 0x7F80, 0xFF80]
    nan = orc.bf16_round(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# ------------------------------------------------------------------------------------------
# hand-worked single groups and the tiny forward
# ------------------------------------------------------------------------------------------
def _group_case(case):
    packed = np.zeros((1, 16), dtype=np.uint8)
    b = int(case["bytes_hex"], 16)
    if case["byte_fill"].startswith("all"):
        packed[:] = b
    else:
        packed[0, 0] = b
    scales = np.array([[case["scale"]]], dtype=np.uint8)
    x = np.zeros(32, dtype=np.float32)
    if case["x"].startswith("1.0 everywhere"):
        x[:] = 1.0
    elif case["x"] == "one-hot at c = 1":
        x[1] = 1.0
    elif case["x"] == "one-hot at c = 0":
        x[0] = 1.0
    else:
        x[0] = x[1] = 1.0
    return x, packed, scales


@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_single_group_examples(orc, acc):
    for case in _golden("hand_examples.json")["single_group"]:
        x, p, s = _group_case(case)
        y = orc.mxfp4_matvec(x, p, s, acc=acc)
        assert y[0] == case["expected"], case["name"]


@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_tiny_forward_s4(orc, acc):
    c = _golden("hand_examples.json")["tiny_forward"]
    H, I = c["H"], c["I"]
    ex = S.ExpertBytes(
        w1_packed=np.full((I, H // 2), int(c["w1_w3_byte"], 16), np.uint8),
        w1_scale=np.full((I, H // 32), c["scale"], np.uint8),
        w3_packed=np.full((I, H // 2), int(c["w1_w3_byte"], 16), np.uint8),
        w3_scale=np.full((I, H // 32), c["scale"], np.uint8),
        w2_packed=np.full((H, I // 2), int(c["w2_byte"], 16), np.uint8),
        w2_scale=np.full((H, I // 32), c["scale"], np.uint8),
    )
    x = np.full(H, int(c["x_bf16_hex"], 16), np.uint16)
    h, g, u, d = orc.expert_forward(x, ex, acc=acc, want_hidden=True)
    assert np.all(g == 4.0) and np.all(u == 4.0)
    assert np.all(h == int(c["h_bf16_hex"], 16))
    assert np.all(d == c["d"])
    pool = {n: np.stack([a, a]) for n, a in zip(S.TENSOR_NAMES, ex.tensors())}
    y, drops = orc.moe_forward(pool, x[None, :], np.array([[0, 1]], np.int32),
                               np.array([c["gates"]], np.float32), acc=acc)
    assert drops == 0 and np.all(y == c["y"])


# ------------------------------------------------------------------------------------------
# brute force on tiny shapes
# ------------------------------------------------------------------------------------------
def _tiny_pool(seed, E, H, I, nan_scales=True):
    exps = [S.expert_bytes(seed, 0, e, H, I) for e in range(E)]
    pool = {n: np.stack([getattr(ex, n) for ex in exps]) for n in S.TENSOR_NAMES}
    if nan_scales:
        # a few NaN scale bytes (255) zero their groups
        pool["w1_scale"][0, 0, 0] = 255
        pool["w2_scale"][1, 2, 0] = 255
        pool["w3_scale"][2, 1, -1] = 255
    return pool


def _brute_force_expert(pool, e, xf64, h_bits):
    W1 = dequant64(pool["w1_packed"][e], pool["w1_scale"][e])
    W3 = dequant64(pool["w3_packed"][e], pool["w3_scale"][e])
    W2 = dequant64(pool["w2_packed"][e], pool["w2_scale"][e])
    g = W1 @ xf64
    u = W3 @ xf64
    v = g / (1.0 + np.exp(-g)) * u
    d = W2 @ bits_to_f(h_bits)
    return g, u, v, d


@pytest.mark.parametrize("H,I", [(32, 32), (64, 96), (96, 64)])
@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_brute_force_tiny(orc, H, I, acc):
    E, k, T = 8, 3, 5
    pool = _tiny_pool(1000 + H + I, E, H, I)
    x = S.normal_bf16(7, S.P_X, 0, (T, H))
    idx, gates = S.uniform_routing(11, T, E, k)
    y, drops = orc.moe_forward(pool, x, idx, gates, acc=acc)
    assert drops == 0
    y_ref = np.zeros((T, H))
    for t in range(T):
        xf = bits_to_f(x[t])
        for j in range(k):
            e = int(idx[t, j])
            ex = S.ExpertBytes(*[pool[n][e] for n in S.TENSOR_NAMES])
            h, g, u, d = orc.expert_forward(x[t], ex, acc=acc, want_hidden=True)
            g64, u64, v64, d64 = _brute_force_expert(pool, e, xf, h)
            scale_g = np.max(np.abs(g64)) + 1e-30
            assert np.max(np.abs(g - g64)) <= 1e-6 * scale_g
            assert np.max(np.abs(u - u64)) <= 1e-6 * (np.max(np.abs(u64)) + 1e-30)
            # h = bf16(silu(g) * u): against the exact value built from the oracle's own g and u
            # (the float exponential inside silu is the float nearest to exp(-g))
            # (g and u were pinned above), h may miss the exact rounding only next to a midpoint
            g64o, u64o = g.astype(np.float64), u.astype(np.float64)
            v = g64o / (1.0 + np.exp(-g64o)) * u64o
            hf = bits_to_f(h)
            want = bf16_rne_from64(v)
            for r in np.nonzero(hf != want)[0]:
                if abs(v[r]) < 2.0 ** -100:
                    # for g < -88.7 exp(-g) overflows float32, so silu(g) is -0 there
                    assert abs(hf[r] - v[r]) <= 2.0 ** -100
                    continue
                ulp = 2.0 ** (math.frexp(v[r])[1] - 8)
                mid = math.floor(v[r] / ulp) * ulp + ulp / 2
                assert abs(v[r] - mid) <= 1e-6 * abs(v[r]), (t, j, r)
            assert np.max(np.abs(d - d64)) <= 1e-6 * (np.max(np.abs(d64)) + 1e-30)
            y_ref[t] += float(gates[t, j]) * d64
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel <= 1e-6


def test_nan_scale_zeroes_only_its_group(orc):
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (4, 48), dtype=np.uint8)  # K = 96, 3 groups
    scales = rng.integers(118, 131, (4, 3), dtype=np.uint8)
    x = rng.standard_normal(96).astype(np.float32)
    y0 = orc.mxfp4_matvec(x, packed, scales, acc="f64")
    s2 = scales.copy()
    s2[1, 1] = 255
    y1 = orc.mxfp4_matvec(x, packed, s2, acc="f64")
    W = dequant64(packed, scales)
    contrib = W[1, 32:64] @ x[32:64].astype(np.float64)
    assert np.array_equal(np.delete(y0, 1), np.delete(y1, 1))
    assert abs(float(y1[1]) - (float(y0[1]) - contrib)) <= 1e-6 * (abs(float(y0[1])) + abs(contrib))


# ------------------------------------------------------------------------------------------
# invariants (exact)
# ------------------------------------------------------------------------------------------
def _small_case(seed=5, E=6, H=64, I=96, T=3, k=4):
    pool = _tiny_pool(seed, E, H, I, nan_scales=False)
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    idx, gates = S.uniform_routing(seed, T, E, k)
    return pool, x, idx, gates


@pytest.mark.parametrize("acc", ["f32", "f64"])
@pytest.mark.parametrize("which", ["w2_scale", "w3_scale"])
def test_scale_plus_one_doubles_y(orc, acc, which):
    pool, x, idx, gates = _small_case()
    y, _ = orc.moe_forward(pool, x, idx, gates, acc=acc)
    p2 = dict(pool)
    p2[which] = pool[which] + 1
    y2, _ = orc.moe_forward(p2, x, idx, gates, acc=acc)
    assert np.array_equal(y2, 2.0 * y)


@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_zero_w1_gives_zero(orc, acc):
    pool, x, idx, gates = _small_case()
    pool["w1_packed"] = np.zeros_like(pool["w1_packed"])
    y, _ = orc.moe_forward(pool, x, idx, gates, acc=acc)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_zero_gate_contributes_nothing(orc, acc):
    pool, x, idx, gates = _small_case(k=3)
    g0 = gates.copy()
    g0[:, 1] = 0.0
    y, _ = orc.moe_forward(pool, x, idx, g0, acc=acc)
    y2, _ = orc.moe_forward(pool, x, idx[:, [0, 2]], g0[:, [0, 2]], acc=acc)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_same_expert_everywhere_gives_d(orc, acc):
    pool, x, _, _ = _small_case(T=1, k=16)
    idx = np.full((1, 16), 2, np.int32)
    _, gates = S.uniform_routing(9, 1, 16, 16)
    y, _ = orc.moe_forward(pool, x, idx, gates, acc=acc)
    ex = S.ExpertBytes(*[pool[n][2] for n in S.TENSOR_NAMES])
    d = orc.expert_forward(x[0], ex, acc=acc)
    # gates sum to 1 within float32 rounding of 16 terms
    assert np.all(np.abs(y[0] - d) <= 2.0 ** -19 * np.abs(d))


def test_permutation_invariance(orc):
    pool, x, idx, gates = _small_case(T=4, k=6)
    rng = np.random.default_rng(17)
    y64, _ = orc.moe_forward(pool, x, idx, gates, acc="f64")
    y32, _ = orc.moe_forward(pool, x, idx, gates, acc="f32")
    for _ in range(4):
        perm = rng.permutation(idx.shape[1])
        p64, _ = orc.moe_forward(pool, x, idx[:, perm], gates[:, perm], acc="f64")
        p32, _ = orc.moe_forward(pool, x, idx[:, perm], gates[:, perm], acc="f32")
        assert np.count_nonzero(p64 != y64) == 0
        assert np.linalg.norm(p32 - y32) <= 1e-6 * np.linalg.norm(y32)


def test_dropped_slots_are_counted_and_contribute_nothing(orc):
    pool, x, idx, gates = _small_case(E=6, T=3, k=4)
    bad = idx.copy()
    bad[0, 1] = -1
    bad[2, 3] = 6
    y, drops = orc.moe_forward(pool, x, bad, gates, acc="f32")
    assert drops == 2
    g2 = gates.copy()
    g2[0, 1] = 0.0
    g2[2, 3] = 0.0
    y_ref, d0 = orc.moe_forward(pool, x, idx, g2, acc="f32")
    assert d0 == 0 and np.array_equal(y, y_ref)


def _edge_expert(seed, H, I):
    """An expert with the format's edge cases: NaN scale bytes (255), rows and scattered
    nibbles of code 8 (-0), and the extreme scale bytes 2 and 252 over groups of zero codes
    (so nothing overflows)."""
    ex = S.expert_bytes(seed, 0, 0, H, I)
    rng = np.random.default_rng(seed)
    for name in ("w1", "w3", "w2"):
        p = getattr(ex, name + "_packed")
        sc = getattr(ex, name + "_scale")
        sc[rng.random(sc.shape) < 0.05] = 255
        sc[rng.random(sc.shape) < 0.03] = 2
        p[1, :] = 0x88
        m = rng.random(p.shape) < 0.05
        p[m] = (p[m] & 0xF0) | 0x08
        r, g = 2, 1
        p[r, 16 * g:16 * g + 16] = 0x80
        sc[r, g] = 252
    return ex


@pytest.mark.parametrize("acc", ["f32", "f64"])
@pytest.mark.parametrize("act", ["swiglu", ("situ", 4.0, 25.0)])
@pytest.mark.parametrize("n", [1, 7, 33])
def test_expert_forward_many_equals_per_token(orc, acc, act, n):
    """The expert-major oracle (one expert on n activations, the tokens side by side in the
    innermost loops) gives every token exactly what the per-token oracle gives it."""
    H, I = 96, 128
    ex = _edge_expert(40 + n, H, I)
    x = S.normal_bf16(41 + n, S.P_X, 0, (n, H))
    x[0, 3] = 0x8000  # -0
    x[n - 1, 5] = 0x0000
    d = orc.expert_forward_many(x, ex, acc=acc, act=act)
    assert np.all(np.isfinite(d))
    for t in range(n):
        want = orc.expert_forward(x[t], ex, acc=acc, act=act)
        assert np.array_equal(d[t].view(np.uint32), want.view(np.uint32)), t


def test_expert_forward_many_full_shape(orc):
    H, I = S.H_K3, S.I_K3
    ex = S.expert_bytes(91, 0, 5, H, I)
    x = S.normal_bf16(91, S.P_X, 0, (5, H))
    d = orc.expert_forward_many(x, ex)
    for t in range(5):
        assert np.array_equal(d[t].view(np.uint32), orc.expert_forward(x[t], ex).view(np.uint32)), t


def test_fp32_oracle_noise_floor_full_size(orc):
    """The verdict (fp32) oracle against its fp64 self-check at the real expert shape."""
    H, I, E, k = S.H_K3, S.I_K3, 4, 4
    pool = {n: np.stack([getattr(S.expert_bytes(77, 0, e, H, I), n) for e in range(E)])
            for n in S.TENSOR_NAMES}
    x = S.normal_bf16(77, S.P_X, 0, (1, H))
    idx = np.arange(k, dtype=np.int32)[None, :]
    _, gates = S.uniform_routing(77, 1, k, k)
    y32, _ = orc.moe_forward(pool, x, idx, gates, acc="f32")
    y64, _ = orc.moe_forward(pool, x, idx, gates, acc="f64")
    rel = np.linalg.norm(y32 - y64) / np.linalg.norm(y64)
    assert rel <= 1e-6, rel


# ------------------------------------------------------------------------------------------
# fixed 64-way reduction
# ------------------------------------------------------------------------------------------
def test_sum64_exact_on_integers_and_bounded_otherwise(orc):
    rng = np.random.default_rng(1)
    a = rng.integers(-1000, 1000, 3584).astype(np.float64)
    b = rng.integers(-1000, 1000, 3584).astype(np.float64)
    assert orc.sum64(a, b) == float(np.sum(a.astype(np.int64) * b.astype(np.int64)))
    a = rng.standard_normal(3584)
    b = rng.standard_normal(3584)
    prods = a * b
    exact = math.fsum(prods)
    bound = 3584 * 2.0 ** -53 * math.fsum(np.abs(prods))
    assert abs(orc.sum64(a, b) - exact) <= bound


# ------------------------------------------------------------------------------------------
# router
# ------------------------------------------------------------------------------------------
def _router_case(T=6, E=128, H=512, seed=21, bias_std=0.01):
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    W = S.normal_bf16(seed, S.P_WR, 0, (E, H), std=0.02 * math.sqrt(3584 / H))
    b = S.normal_f32(seed, S.P_BIAS, 0, (E,), std=bias_std)
    return x, W, b


def test_router_logits_are_the_rounded_exact_dot(orc):
    x, W, b = _router_case(T=4, E=896, H=3584)
    _, _, lg, sc = orc.route(x, W, b, 16, want_scores=True)
    xf, wf = bits_to_f(x), bits_to_f(W)
    for t in range(4):
        prods = xf[t][None, :] * wf  # exact in float64
        exact = np.array([math.fsum(p) for p in prods], dtype=np.float64)
        assert np.array_equal(lg[t], exact.astype(np.float32))
        assert np.array_equal(sc[t], (1.0 / (1.0 + np.exp(-lg[t].astype(np.float64)))).astype(np.float32))


def test_router_no_bias_is_stable_argsort_of_scores(orc):
    x, W, _ = _router_case(T=16, E=256, H=512)
    idx, gates, lg, sc = orc.route(x, W, None, 16, want_scores=True)
    for t in range(16):
        want = np.argsort(-sc[t], kind="stable")[:16]
        assert np.array_equal(idx[t], want)
        # sigmoid is monotone: the same set is the top-16 logits
        assert set(idx[t]) == set(np.argsort(-lg[t], kind="stable")[:16]) or \
            len(np.unique(sc[t])) < len(sc[t])


def test_router_with_bias_is_stable_argsort_of_selection_scores(orc):
    x, W, b = _router_case(T=16, E=256, H=512, bias_std=0.05)
    idx, gates, lg, sc = orc.route(x, W, b, 16, want_scores=True)
    for t in range(16):
        c = (sc[t] + b).astype(np.float32)
        assert np.array_equal(idx[t], np.argsort(-c, kind="stable")[:16])


def test_router_full_permutation_when_k_equals_e(orc):
    x, W, b = _router_case(T=3, E=64, H=256)
    idx, gates = orc.route(x, W, b, 64)
    for t in range(3):
        assert sorted(idx[t].tolist()) == list(range(64))


def test_router_exact_tie_goes_to_lower_index(orc):
    x, W, b = _router_case(T=2, E=32, H=256)
    W = W.copy()
    W[9] = W[5]
    b = b.copy()
    b[5] = b[9] = 10.0
    idx, _ = orc.route(x, W, b, 4)
    assert idx[0, 0] == 5 and idx[0, 1] == 9 and idx[1, 0] == 5 and idx[1, 1] == 9


def test_router_bias_steers_selection_only(orc):
    """Combine weights come from the unbiased scores: changing the bias of experts that stay
    unselected leaves idx and gates bit-identical (README section 9; invariant 5 of the
    README's list of invariants)."""
    x, W, b = _router_case(T=8, E=128, H=512)
    idx, gates, _, sc = orc.route(x, W, b, 16, want_scores=True)
    for t in range(8):
        b2 = b.copy()
        others = np.setdiff1d(np.arange(128), idx[t])
        b2[others] -= 1.0
        i2, g2 = orc.route(x[t:t + 1], W, b2, 16)
        assert np.array_equal(i2[0], idx[t]) and np.array_equal(g2[0], gates[t])
        # and the gates are the renormalised unbiased scores of the chosen experts
        s = sc[t, idx[t]]
        assert np.all(np.abs(gates[t] - s / s.sum(dtype=np.float64)) <= 4e-7)


def test_router_renorm_and_scale(orc):
    x, W, b = _router_case(T=4, E=64, H=256)
    idx, g1, _, sc = orc.route(x, W, b, 8, renorm=1, routed_scale=1.0, want_scores=True)
    assert np.all(np.abs(g1.sum(axis=1, dtype=np.float64) - 1.0) <= 8 * 2.0 ** -24)
    i0, g0 = orc.route(x, W, b, 8, renorm=0, routed_scale=1.0)
    assert np.array_equal(i0, idx)
    assert np.array_equal(g0, np.take_along_axis(sc, idx, axis=1))
    _, g25 = orc.route(x, W, b, 8, renorm=1, routed_scale=2.5)
    assert np.array_equal(g25, (g1 * np.float32(2.5)).astype(np.float32))


# ------------------------------------------------------------------------------------------
# RMSNorm and residual
# ------------------------------------------------------------------------------------------
def test_rmsnorm_constant_vector_closed_form(orc):
    eps = np.float32(1e-6)
    for a_bits in (0x3F80, 0x4049, 0xBE00, 0x3A80, 0x4500):
        a = float(S.bf16_bits_to_f32(np.uint16(a_bits)))
        x = np.full((1, 3584), a_bits, np.uint16)
        out = orc.rmsnorm_bf16(x, float(eps))
        inv = np.float32(1.0 / math.sqrt(a * a + float(eps)))
        want = S.f32_to_bf16_bits(np.float32(a) * inv)
        assert np.all(out == want), hex(a_bits)


def test_rmsnorm_random_against_fsum(orc):
    x = S.normal_bf16(3, S.P_X, 0, (8, 3584))
    out = orc.rmsnorm_bf16(x, 1e-6)
    xf = bits_to_f(x)
    for t in range(8):
        ss = math.fsum(xf[t] * xf[t])
        inv = np.float32(1.0 / math.sqrt(ss / 3584.0 + float(np.float32(1e-6))))
        want = S.f32_to_bf16_bits((xf[t].astype(np.float32) * inv).astype(np.float32))
        assert np.array_equal(out[t], want)


def test_residual_add(orc):
    x = S.normal_bf16(4, S.P_X, 0, (3, 64))
    y = np.random.default_rng(4).standard_normal((3, 64)).astype(np.float32)
    out = orc.residual_add_bf16(x, y)
    want = S.f32_to_bf16_bits((S.bf16_bits_to_f32(x) + y).astype(np.float32))
    assert np.array_equal(out, want)


# ------------------------------------------------------------------------------------------
# SiTU-GLU (kimi-k3-in-c README Part II section 9, the routed-expert loop's activation
# listing; caps b1 = 4, b2 = 25 from the config header)
# ------------------------------------------------------------------------------------------
SITU = ("situ", 4.0, 25.0)


def test_situ_saturates_at_the_cap_product(orc):
    """The engine's self-test prints |out| = 100.000 = b1 * b2 for a saturated input; the
    float tanh of a large argument is 1 and the sigmoid of a large gate is 1."""
    g = np.array([100.0, 60.0, 1e4, 3e4], np.float32)
    u = np.array([1e4, 1e3, 1e5, 2e3], np.float32)
    assert np.all(orc.glu(g, u, SITU) == 100.0)
    assert np.all(orc.glu(g, -u, SITU) == -100.0)
    assert np.all(orc.glu(g, u, ("situ", 2.0, 3.0)) == 6.0)


def test_situ_bounded_by_the_cap_product(orc):
    rng = np.random.default_rng(5)
    g = (rng.standard_normal(200000) * rng.choice([0.1, 3.0, 100.0], 200000)).astype(np.float32)
    u = (rng.standard_normal(200000) * rng.choice([0.1, 30.0, 1000.0], 200000)).astype(np.float32)
    h = orc.glu(g, u, SITU)
    assert np.all(np.isfinite(h)) and np.all(np.abs(h) <= 100.0)


def test_situ_zero_gate_and_odd_in_the_up_projection(orc):
    rng = np.random.default_rng(6)
    g = (rng.standard_normal(50000) * 5).astype(np.float32)
    u = (rng.standard_normal(50000) * 50).astype(np.float32)
    assert np.all(orc.glu(np.zeros_like(g), u, SITU) == 0.0)
    # tanh and the fp32 quotient are odd, so flipping u flips h exactly
    assert np.array_equal(orc.glu(g, -u, SITU), -orc.glu(g, u, SITU))


def test_situ_tends_to_swiglu_for_large_caps(orc):
    """b * tanh(q / b) -> q as b -> infinity, so the activation becomes silu(g) * u."""
    rng = np.random.default_rng(7)
    g = (rng.standard_normal(50000) * 4).astype(np.float32)
    u = (rng.standard_normal(50000) * 4).astype(np.float32)
    big = orc.glu(g, u, ("situ", 1e7, 1e7))
    sw = orc.glu(g, u, "swiglu")
    assert np.allclose(big, sw, rtol=2e-6, atol=1e-37)


def test_situ_within_the_pages_tolerance_of_the_exact_value(orc):
    """The engine checks this kernel at atol 1e-5, rtol 1e-4; the oracle's fp32 rounding
    steps stay far inside that against the exact value (float64 math)."""
    rng = np.random.default_rng(8)
    g = (rng.standard_normal(100000) * 6).astype(np.float32)
    u = (rng.standard_normal(100000) * 60).astype(np.float32)
    h = orc.glu(g, u, SITU).astype(np.float64)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    exact = 4.0 * np.tanh(g64 / 4.0) / (1.0 + np.exp(-g64)) * (25.0 * np.tanh(u64 / 25.0))
    assert np.allclose(h, exact, atol=1e-5, rtol=1e-4)
    assert np.max(np.abs(h - exact) / (np.abs(exact) + 1e-30)) < 1e-5


def test_situ_rejects_bad_caps(orc):
    g = np.ones(4, np.float32)
    for b1, b2 in ((0.0, 25.0), (4.0, -1.0), (float("inf"), 25.0), (4.0, float("nan"))):
        with pytest.raises(ValueError):
            orc.glu(g, g, ("situ", b1, b2))


@pytest.mark.parametrize("acc", ["f32", "f64"])
def test_situ_expert_against_brute_force(orc, acc):
    """A whole expert with SiTU-GLU on tiny shapes: h equals bf16 of the activation of the
    oracle's own g and u, and d, y follow numpy's float64 algebra."""
    E, H, I, k, T = 6, 64, 96, 3, 4
    pool = _tiny_pool(4242, E, H, I)
    x = S.normal_bf16(9, S.P_X, 0, (T, H))
    idx, gates = S.uniform_routing(13, T, E, k)
    y, drops = orc.moe_forward(pool, x, idx, gates, acc=acc, act=SITU)
    assert drops == 0
    y_ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            ex = S.ExpertBytes(*[pool[n][e] for n in S.TENSOR_NAMES])
            h, g, u, d = orc.expert_forward(x[t], ex, acc=acc, want_hidden=True, act=SITU)
            assert np.array_equal(bits_to_f(h), bf16_rne_from64(orc.glu(g, u, SITU)))
            d64 = dequant64(pool["w2_packed"][e], pool["w2_scale"][e]) @ bits_to_f(h)
            assert np.max(np.abs(d - d64)) <= 1e-6 * (np.max(np.abs(d64)) + 1e-30)
            y_ref[t] += float(gates[t, j]) * d64
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) <= 1e-6
    # the SiTU forward differs from the SwiGLU one (the option reaches the activation)
    y_sw, _ = orc.moe_forward(pool, x, idx, gates, acc=acc)
    assert not np.allclose(y, y_sw)


# ------------------------------------------------------------------------------------------
# Latent MoE block (kimi-k3-in-c README, Part II section 9, the k3_moe listing)
# ------------------------------------------------------------------------------------------
def _latent_case(seed, T=3, D=96, L=64, I=64, n_shared=2, E=6, k=3):
    S_ = n_shared * I
    w = S.latent_inputs(seed, 0, D, L, S_, E)
    pool = _tiny_pool(seed, E, L, I, nan_scales=False)
    x = S.normal_bf16(seed, S.P_X, 0, (T, D))
    return w, pool, x, k


def _bf16_round64(v):
    return bf16_rne_from64(v)


def _mx_row(codes, scale_bytes):
    """Packed nibbles (low nibble = even element) and scale bytes of one row."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None], np.asarray(scale_bytes, np.uint8)[None]


def test_contract_matvec_exact_on_integers(orc):
    """The contract's MXFP4 matmul on integer-valued data is exact whatever the order: every row
    equals its integer dot product (a transposed, dropped or misplaced term changes it)."""
    rng = np.random.default_rng(8)
    rows, K = 5, 256
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    vals = np.array([orc.e2m1(int(c)) for c in range(16)])
    W = vals[codes]
    x = rng.integers(-4, 5, K).astype(np.float32)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((rows, K // 32), 128, dtype=np.uint8)  # 2.0
    y = orc.mxfp4_matvec_contract(x, packed, scales)
    assert np.array_equal(y, (2.0 * (W @ x.astype(np.float64))).astype(np.float32))


def test_contract_matvec_skips_nan_scales_and_sums_groups_in_order(orc):
    # a scale byte of 255 drops its group, whatever its nibbles
    codes = [2] * 64  # 1.0 everywhere
    x = np.ones(64, dtype=np.float32)
    p, sc = _mx_row(codes, [127, 255])
    assert orc.mxfp4_matvec_contract(x, p, sc)[0] == 32.0
    # group terms 1, 2^60, -2^60, 1: the listing adds them in sequence, ((1 + 2^60) - 2^60) + 1
    # = 1 (the first 1 is lost to rounding), where a pairwise tree gives (1 + 2^60) +
    # (-2^60 + 1) = 0
    K = 128
    codes = np.zeros(K, dtype=np.uint8)
    codes[[0, 32, 64, 96]] = [2, 2, 10, 2]  # 1.0, 1.0, -1.0, 1.0
    p, sc = _mx_row(codes, [127, 187, 187, 127])  # scales 1, 2^60, 2^60, 1
    x = np.ones(K, dtype=np.float32)
    assert orc.mxfp4_matvec_contract(x, p, sc)[0] == 1.0
    assert orc.mxfp4_matvec(x, p, sc, acc="f64")[0] == 0.0


def test_contract_expert_against_float64_algebra(orc):
    """The contract's expert forward (h kept in fp32) against numpy float64 algebra on the
    dequantised weights, rounding g, u and h to fp32 at the same points."""
    H, I = 256, 384
    ex = S.expert_bytes(3, 0, 1, H, I)
    x = S.normal_bf16(3, S.P_X, 0, (H,))
    for act in ("swiglu", ("situ", 4.0, 25.0)):
        d, h = orc.expert_forward_contract(x, ex, act=act, want_hidden=True)
        xf = bits_to_f(x)
        W1 = dequant64(ex.w1_packed, ex.w1_scale)
        W3 = dequant64(ex.w3_packed, ex.w3_scale)
        W2 = dequant64(ex.w2_packed, ex.w2_scale)
        g, u = (W1 @ xf).astype(np.float32), (W3 @ xf).astype(np.float32)
        h_ref = orc.glu(g, u, act)
        assert np.max(np.abs(h - h_ref)) <= 1e-6 * np.max(np.abs(h_ref))
        d_ref = W2 @ h.astype(np.float64)
        assert np.linalg.norm(d - d_ref) / np.linalg.norm(d_ref) < 1e-6
        # the bf16 rounding of h is what separates it from the routed path's arithmetic
        d_bf16 = orc.expert_forward(x, ex, acc="f64", act=act)
        assert not np.array_equal(d, d_bf16)


def test_dense64_exact_on_integers(orc):
    """The contract's bf16 matmul on small integers: every product and partial sum is exact,
    so each row must equal its integer dot product whatever the order (a dropped term, a
    swapped index or a transposed operand changes it)."""
    rng = np.random.default_rng(5)
    rows, K = 7, 1032
    Wi = rng.integers(-8, 9, (rows, K))
    vi = rng.integers(-8, 9, K)
    W = S.f32_to_bf16_bits(Wi.astype(np.float32))
    v = S.f32_to_bf16_bits(vi.astype(np.float32))
    y = orc.dense64_bf16(W, v)
    assert np.array_equal(y, (Wi @ vi).astype(np.float32))
    assert not np.array_equal(orc.dense64_bf16(W[:, ::-1].copy(), v), y)


def test_dense64_within_one_ulp_of_exact_sum(orc):
    """Random bf16 rows: the double sum rounded to float lies within one float ulp of the
    exactly rounded sum of the exact products (math.fsum)."""
    rng = np.random.default_rng(6)
    rows, K = 9, 3584
    W = S.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    v = S.f32_to_bf16_bits(rng.standard_normal(K).astype(np.float32))
    y = orc.dense64_bf16(W, v)
    Wf, vf = bits_to_f(W), bits_to_f(v)
    for r in range(rows):
        exact = np.float32(math.fsum((Wf[r] * vf).tolist()))
        assert abs(float(y[r]) - float(exact)) <= float(np.spacing(np.abs(exact))), r


def test_dense64_fixed_64_way_order(orc):
    """The order of the double sum is the fixed 64-way one: products 2^60, 1 and -2^60 in the
    chunks of partials 0, 1 and 2 fold as (2^60 + -2^60) + 1 = 1, where ascending order (and
    the contract's four interleaved accumulators) lose the 1 to rounding and give 0."""
    K = 512
    Wf = np.zeros(K, dtype=np.float32)
    vf = np.zeros(K, dtype=np.float32)
    Wf[0], vf[0] = 2.0 ** 30, 2.0 ** 30       # chunk 0 -> partial 0
    Wf[8], vf[8] = 1.0, 1.0                   # chunk 1 -> partial 1
    Wf[16], vf[16] = -(2.0 ** 30), 2.0 ** 30  # chunk 2 -> partial 2
    y = orc.dense64_bf16(S.f32_to_bf16_bits(Wf)[None], S.f32_to_bf16_bits(vf))
    assert y[0] == 1.0
    seq = 0.0
    for k in range(K):
        seq += float(Wf[k]) * float(vf[k])
    assert seq == 0.0


def test_latent_block_against_float64_algebra(orc):
    """The whole block recomputed with numpy float64 dense algebra and the pinned pieces
    (router, SiTU-GLU, E2M1/E8M0 decode), rounding to bf16 at the same points."""
    w, pool, x, k = _latent_case(31)
    act = ("situ", 4.0, 25.0)
    out, drops = orc.latent_block(x, w["Wr"], w["bias"], k, w["down"], w["up"], w["sh1"],
                                  w["sh3"], w["sh2"], w["norm_w"], 1e-6, pool, act=act,
                                  act_shared=act, acc="f64")
    assert drops == 0
    idx, gates = orc.route(x, w["Wr"], w["bias"], k)
    f = lambda a: bits_to_f(a)
    down, up, sh1, sh3, sh2 = (f(w[n]) for n in ("down", "up", "sh1", "sh3", "sh2"))
    for t in range(x.shape[0]):
        xt = f(x[t])
        z = _bf16_round64(down @ xt)
        acc = np.zeros(down.shape[0])
        for j in range(k):
            e = int(idx[t, j])
            W1 = dequant64(pool["w1_packed"][e], pool["w1_scale"][e])
            W3 = dequant64(pool["w3_packed"][e], pool["w3_scale"][e])
            W2 = dequant64(pool["w2_packed"][e], pool["w2_scale"][e])
            g, u = (W1 @ z).astype(np.float32), (W3 @ z).astype(np.float32)
            h = _bf16_round64(orc.glu(g, u, act).astype(np.float64))
            acc += float(gates[t, j]) * (W2 @ h)
        ss = math.fsum(acc.astype(np.float32).astype(np.float64) ** 2)
        inv = 1.0 / math.sqrt(ss / len(acc) + 1e-6)
        a = _bf16_round64(acc * inv * w["norm_w"].astype(np.float64))
        o = up @ a
        g, u = (sh1 @ xt).astype(np.float32), (sh3 @ xt).astype(np.float32)
        s_ = _bf16_round64(orc.glu(g, u, act).astype(np.float64))
        ref = o + sh2 @ s_
        rel = np.linalg.norm(out[t] - ref) / np.linalg.norm(ref)
        assert rel < 1e-6, (t, rel)
    out32, _ = orc.latent_block(x, w["Wr"], w["bias"], k, w["down"], w["up"], w["sh1"],
                                w["sh3"], w["sh2"], w["norm_w"], 1e-6, pool, act=act,
                                act_shared=act)
    assert np.linalg.norm(out32 - out) / np.linalg.norm(out) < 1e-4


def test_latent_norm_is_on_the_aggregate(orc):
    """The RMSNorm acts on the weighted sum of the experts: scaling every gate (routed_scale)
    leaves the block's output unchanged up to eps and rounding, while without the norm the
    routed part scales with the gates exactly."""
    w, pool, x, k = _latent_case(37)
    zero = np.zeros_like(w["sh2"])
    common = (w["Wr"], w["bias"], k, w["down"], w["up"], w["sh1"], w["sh3"])
    o1, _ = orc.latent_block(x, *common, w["sh2"], w["norm_w"], 1e-6, pool, routed_scale=1.0)
    o2, _ = orc.latent_block(x, *common, w["sh2"], w["norm_w"], 1e-6, pool, routed_scale=2.0)
    assert np.linalg.norm(o2 - o1) / np.linalg.norm(o1) < 1e-2
    # no norm, no shared experts: doubling the gates doubles the output exactly
    n1, _ = orc.latent_block(x, *common, zero, None, 1e-6, pool, routed_scale=1.0)
    n2, _ = orc.latent_block(x, *common, zero, None, 1e-6, pool, routed_scale=2.0)
    assert np.array_equal(n2, 2.0 * n1)
    assert not np.allclose(n1, o1)


def test_latent_shared_experts_added_unweighted(orc):
    """With the shared down-projection sh2 zeroed the output is exactly the routed part; the
    shared part alone (router bias steering the routed experts elsewhere) is the same for
    any routing."""
    w, pool, x, k = _latent_case(41)
    zero = np.zeros_like(w["sh2"])
    args = (w["Wr"], w["bias"], k, w["down"], w["up"], w["sh1"], w["sh3"])
    full, _ = orc.latent_block(x, *args, w["sh2"], w["norm_w"], 1e-6, pool)
    routed, _ = orc.latent_block(x, *args, zero, w["norm_w"], 1e-6, pool)
    shared = full - routed
    b2 = w["bias"].copy()
    b2[:3] += 10.0  # forces experts 0..2
    full2, _ = orc.latent_block(x, w["Wr"], b2, k, w["down"], w["up"], w["sh1"], w["sh3"],
                                w["sh2"], w["norm_w"], 1e-6, pool)
    routed2, _ = orc.latent_block(x, w["Wr"], b2, k, w["down"], w["up"], w["sh1"], w["sh3"],
                                  zero, w["norm_w"], 1e-6, pool)
    assert not np.allclose(routed, routed2)
    assert np.allclose(full2 - routed2, shared, rtol=1e-5, atol=1e-5 * np.abs(shared).max())


def test_weighted_rmsnorm(orc):
    """Unit weight equals the bf16 RMSNorm on bf16-valued rows; a weight of 2 doubles the
    output exactly; the constant-vector closed form."""
    x = bits_to_f(S.normal_bf16(3, S.P_X, 0, (4, 256))).astype(np.float32)
    xb = S.f32_to_bf16_bits(x)
    one = orc.rmsnorm_w_f32(x, None, 1e-6)
    assert np.array_equal(one, orc.rmsnorm_bf16(xb, 1e-6))
    two = orc.rmsnorm_w_f32(x, np.full(256, 2.0, np.float32), 1e-6)
    assert np.array_equal(bits_to_f(two), 2.0 * bits_to_f(one))
    c = np.full((1, 64), 3.0, np.float32)
    assert np.all(bits_to_f(orc.rmsnorm_w_f32(c, None, 0.0)) == 1.0)
