"""The verdict helpers of the parity tests (tests/cases.py), checked on the CPU: the
tolerances are applied as stated, and the fp64 fallback is taken only where the fp32 oracle
itself lies beyond the tolerance from the fp64 oracle."""
import numpy as np
import pytest

import k3x_synth as S
from cases import (FALLBACKS, MAX_ABS_TOL, REL_L2_TOL, assert_y_close, assert_y_close_oracle,
                   oracle_forward_all, oracle_forward_sampled, token_errors, y_errors)


def _ref(seed=0, shape=(6, 64)):
    return np.random.default_rng(seed).standard_normal(shape)


def test_y_errors_definitions():
    r = _ref()
    y = r.copy()
    y[2, 5] += 0.5
    rel, mx = y_errors(y, r)
    assert rel == pytest.approx(0.5 / np.linalg.norm(r))
    assert mx == pytest.approx(0.5 / np.abs(r).max())
    assert y_errors(r, r) == (0.0, 0.0)


def test_assert_y_close_bounds():
    r = _ref()
    assert_y_close(r * (1 + 0.5 * REL_L2_TOL), r)
    with pytest.raises(AssertionError):
        assert_y_close(r * (1 + 2 * REL_L2_TOL), r)
    y = r.copy()
    y[0, 0] += 2 * MAX_ABS_TOL * np.abs(r).max()  # one large error, tiny L2 share on a big array
    big = np.tile(r, (200, 1))
    yb = big.copy()
    yb[0, 0] = y[0, 0]
    with pytest.raises(AssertionError):
        assert_y_close(yb, big)
    with pytest.raises(AssertionError):
        assert_y_close(np.where(r > 0, np.nan, r), r)


def test_oracle_fallback_only_when_fp32_oracle_is_off():
    r64 = _ref(1)
    noisy32 = r64.copy()
    noisy32[1, 1] += 5 * MAX_ABS_TOL * np.abs(r64).max()  # the fp32 oracle beyond the tolerance
    # a result at the fp64 oracle passes through the fallback
    assert_y_close_oracle(r64, noisy32, lambda: r64)
    # a result far from both fails
    with pytest.raises(AssertionError):
        assert_y_close_oracle(r64 + 0.1, noisy32, lambda: r64)
    # when the fp32 oracle agrees with the fp64 one, no fallback: a miss of the fp32 oracle fails
    with pytest.raises(AssertionError):
        assert_y_close_oracle(noisy32, r64, lambda: r64)
    # a result within tolerance of the fp64 oracle but farther from it than the fp32 oracle
    # is fails: the fallback never accepts a worse result
    big64 = _ref(2, (400, 64))
    scaled32 = big64 * (1 + 3 * REL_L2_TOL)  # fp32 oracle off in rel L2 only (max-abs 3e-4)
    worse = big64.copy()
    worse[0, 0] += 0.8 * MAX_ABS_TOL * np.abs(big64).max()  # within tolerance, past the floor
    assert y_errors(worse, big64)[0] <= REL_L2_TOL and y_errors(worse, big64)[1] <= MAX_ABS_TOL
    with pytest.raises(AssertionError, match="farther than the fp32 oracle"):
        assert_y_close_oracle(worse, scaled32, lambda: big64)
    # every fallback is recorded
    n = len(FALLBACKS)
    assert_y_close_oracle(r64, noisy32, lambda: r64)
    assert len(FALLBACKS) == n + 1 and FALLBACKS[-1][1][1] > MAX_ABS_TOL
    # results within tolerance of the fp32 oracle never consult the fp64 one
    assert_y_close_oracle(r64, r64, lambda: (_ for _ in ()).throw(RuntimeError("not needed")))


def test_token_errors_name_the_worst_token():
    r = _ref(3, (5, 32))
    y = r.copy()
    y[3] *= 1 + 1e-3
    y[1, 7] += 0.25
    rel, t_rel, mx, t_mx = token_errors(y, r)
    assert t_rel == 1 or t_rel == 3
    assert rel == pytest.approx(max(np.linalg.norm(y[t] - r[t]) / np.linalg.norm(r[t]) for t in range(5)))
    assert t_mx == int(np.argmax([np.abs(y[t] - r[t]).max() / np.abs(r[t]).max() for t in range(5)]))
    assert mx == pytest.approx(np.abs(y[t_mx] - r[t_mx]).max() / np.abs(r[t_mx]).max())


@pytest.mark.parametrize("act", ["swiglu", ("situ", 4.0, 25.0)])
def test_expert_major_reference_equals_per_token_oracle(orc, act):
    """The whole-tensor reference of the full-size parity tests (experts walked one by one,
    per-slot outputs kept, slot-order combine) equals the oracle's per-token forward, with
    duplicates and dropped slots."""
    E, H, I, T, k, seed = 7, 64, 96, 23, 4, 515
    pool = S.host_pool(seed, 0, E, H, I)
    x = S.normal_bf16(seed, S.P_X, 0, (T, H))
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[3, 1] = E + 2
    idx[5, 0] = -1
    _, gates = S.uniform_routing(seed, T, k, k)
    for acc in ("f32", "f64"):
        want, drops = orc.moe_forward(pool, x, idx, gates, acc=acc, act=act)
        assert drops == 2
        got = oracle_forward_all(orc, seed, 0, H, I, x, idx, gates, E=E, acc=acc, act=act)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), acc
        some = oracle_forward_sampled(orc, seed, 0, H, I, x, idx, gates, [0, 3, 22], E=E, acc=acc, act=act)
        assert np.array_equal(some.view(np.uint32), want[[0, 3, 22]].view(np.uint32)), acc
