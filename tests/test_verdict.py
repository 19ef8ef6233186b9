"""The verdict helpers of the parity tests (tests/cases.py), checked on the CPU: the
tolerances are applied as stated, and the fp64 fallback is taken only where the fp32 oracle
itself lies beyond the tolerance from the fp64 oracle."""
import numpy as np
import pytest

from cases import MAX_ABS_TOL, REL_L2_TOL, assert_y_close, assert_y_close_oracle, y_errors


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
    # results within tolerance of the fp32 oracle never consult the fp64 one
    assert_y_close_oracle(r64, r64, lambda: (_ for _ in ()).throw(RuntimeError("not needed")))
