"""Shared helpers of the parity tests: seeded cases, oracle references and the verdict
metrics.  Inputs come from k3x_synth only; expected values come from the oracle only."""
from __future__ import annotations

import numpy as np

import k3x_synth as S

# verdict tolerances for y (floating point): relative L2 and max-abs relative to max|y_ref|
REL_L2_TOL = 1e-4
MAX_ABS_TOL = 1e-3


def y_errors(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    rel_l2 = float(np.linalg.norm(y - r) / max(np.linalg.norm(r), 1e-300))
    max_abs = float(np.max(np.abs(y - r)) / max(np.max(np.abs(r)), 1e-300)) if r.size else 0.0
    return rel_l2, max_abs


def assert_y_close(y, y_ref, what=""):
    rel_l2, max_abs = y_errors(y, y_ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert rel_l2 <= REL_L2_TOL and max_abs <= MAX_ABS_TOL, \
        f"{what}: rel L2 {rel_l2:.3e} (tol {REL_L2_TOL}), max abs {max_abs:.3e} (tol {MAX_ABS_TOL})"
    return rel_l2, max_abs


def assert_y_close_oracle(y, y_ref32, y_ref64_fn, what=""):
    """Verdict against the oracle in its fp32 arithmetic.  The oracle's fp32 sums are one
    rounding of the definition and its fp64 sums another; where the fp32 one already lies
    beyond the tolerance from the fp64 one (a bf16 rounding of a large h that falls the other
    way, amplified by W2), the same tolerance is applied against the fp64 oracle instead."""
    r32 = y_errors(y, y_ref32)
    if r32[0] <= REL_L2_TOL and r32[1] <= MAX_ABS_TOL:
        assert np.all(np.isfinite(y)), f"{what}: non-finite output"
        return r32
    y_ref64 = y_ref64_fn()
    floor = y_errors(y_ref32, y_ref64)
    assert floor[0] > REL_L2_TOL or floor[1] > MAX_ABS_TOL, (
        f"{what}: rel L2 {r32[0]:.3e}, max abs {r32[1]:.3e} against the fp32 oracle, whose own "
        f"distance to the fp64 oracle is only {floor[0]:.3e} / {floor[1]:.3e}")
    return assert_y_close(y, y_ref64, f"{what} [fp64 oracle; fp32 oracle off by {floor[0]:.2e} / {floor[1]:.2e}]")


def oracle_forward_sampled(orc, seed, layer, H, I, x_bits, idx, gates, tokens, E=None,
                           acc="f32", cache=None, act="swiglu"):
    """Oracle y for the listed tokens, regenerating on the host only the experts they use.
    Slots with expert ids outside [0, E) contribute nothing."""
    tokens = list(tokens)
    k = idx.shape[1]
    d = np.zeros((len(tokens), k, H), dtype=np.float32)
    valid = np.zeros((len(tokens), k), dtype=np.uint8)
    need = {}
    for ti, t in enumerate(tokens):
        for j in range(k):
            e = int(idx[t, j])
            if E is not None and not (0 <= e < E):
                continue
            need.setdefault(e, []).append((ti, j))
    for e, uses in need.items():
        key = (seed, layer, e)
        ex = cache.get(key) if cache is not None else None
        if ex is None:
            ex = S.expert_bytes(seed, layer, e, H, I)
            if cache is not None:
                cache[key] = ex
        for ti, j in uses:
            d[ti, j] = orc.expert_forward(x_bits[tokens[ti]], ex, acc=acc, act=act)
            valid[ti, j] = 1
    return orc.combine(gates[tokens], d, valid, acc=acc)
