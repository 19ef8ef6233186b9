"""Shared helpers of the parity tests: seeded cases, oracle references and the verdict
metrics.  Inputs come from k3x_synth only; expected values come from the oracle only."""
from __future__ import annotations

import collections
import concurrent.futures as cf

import numpy as np

import k3x_synth as S

# verdict tolerances for y (floating point): relative L2 and max-abs relative to max|y_ref|
REL_L2_TOL = 1e-4
MAX_ABS_TOL = 1e-3

# Every use of the fp64 fallback of assert_y_close_oracle, in order: (what, errors of the
# result against the fp32 oracle, distance of the fp32 oracle to the fp64 one, errors of the
# result against the fp64 oracle).  The session summary (conftest.py) reports them.
FALLBACKS: list = []


def y_errors(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    rel_l2 = float(np.linalg.norm(y - r) / max(np.linalg.norm(r), 1e-300))
    max_abs = float(np.max(np.abs(y - r)) / max(np.max(np.abs(r)), 1e-300)) if r.size else 0.0
    return rel_l2, max_abs


def token_errors(y, y_ref):
    """Per-token diagnostics over a [T][H] output: (worst rel L2 of one token, its index,
    worst max-abs of one token relative to that token's own max|y_ref|, its index)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    diff = y - r
    rel = np.linalg.norm(diff, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    mx = np.max(np.abs(diff), axis=1) / np.maximum(np.max(np.abs(r), axis=1), 1e-300)
    return float(rel.max()), int(rel.argmax()), float(mx.max()), int(mx.argmax())


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
    way, amplified by W2), the result is checked against the fp64 oracle instead, and must
    then be at least as close to it as the fp32 oracle is, on both measures.  Each such use
    is printed and recorded in FALLBACKS."""
    r32 = y_errors(y, y_ref32)
    if r32[0] <= REL_L2_TOL and r32[1] <= MAX_ABS_TOL:
        assert np.all(np.isfinite(y)), f"{what}: non-finite output"
        return r32
    y_ref64 = y_ref64_fn()
    floor = y_errors(y_ref32, y_ref64)
    r64 = y_errors(y, y_ref64)
    FALLBACKS.append((what, r32, floor, r64))
    print(f"FP64 FALLBACK #{len(FALLBACKS)} {what}: against fp32 oracle {r32[0]:.3e} / {r32[1]:.3e}; "
          f"fp32 oracle vs fp64 {floor[0]:.3e} / {floor[1]:.3e}; against fp64 oracle "
          f"{r64[0]:.3e} / {r64[1]:.3e}", flush=True)
    assert floor[0] > REL_L2_TOL or floor[1] > MAX_ABS_TOL, (
        f"{what}: rel L2 {r32[0]:.3e}, max abs {r32[1]:.3e} against the fp32 oracle, whose own "
        f"distance to the fp64 oracle is only {floor[0]:.3e} / {floor[1]:.3e}")
    assert r64[0] <= floor[0] and r64[1] <= floor[1], (
        f"{what}: {r64[0]:.3e} / {r64[1]:.3e} from the fp64 oracle, farther than the fp32 oracle "
        f"({floor[0]:.3e} / {floor[1]:.3e})")
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


def oracle_forward_all(orc, seed, layer, H, I, x_bits, idx, gates, E=None, acc="f32",
                       act="swiglu", log=None):
    """Oracle y for every token, walking the experts one by one as a prefill does: each
    used expert's bytes are regenerated once on the host (a few experts ahead, in worker
    threads) and applied to all the slots routed to it (orc.expert_forward_many, equal to the
    per-token oracle bit for bit); the per-slot outputs are kept, so the combine runs in slot
    order.  Slots with expert ids outside [0, E) contribute nothing."""
    T, k = idx.shape
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    d = np.zeros((T * k, H), dtype=np.float32)
    valid = np.zeros(T * k, dtype=np.uint8)
    keep = flat >= 0 if E is None else (flat >= 0) & (flat < E)
    slots = np.nonzero(keep)[0]
    order = slots[np.argsort(flat[slots], kind="stable")]
    experts, starts = np.unique(flat[order], return_index=True)
    bounds = list(starts) + [len(order)]
    ahead = 4
    with cf.ThreadPoolExecutor(max_workers=ahead) as pool:
        pending = collections.deque()
        nxt = 0
        for i, e in enumerate(experts):
            while nxt < len(experts) and nxt < i + ahead:
                pending.append(pool.submit(S.expert_bytes, seed, layer, int(experts[nxt]), H, I))
                nxt += 1
            ex = pending.popleft().result()
            sl = order[bounds[i]:bounds[i + 1]]
            d[sl] = orc.expert_forward_many(x_bits[sl // k], ex, acc=acc, act=act)
            valid[sl] = 1
            if log is not None and (i + 1) % 128 == 0:
                log(f"  oracle ({acc}): {i + 1} of {len(experts)} experts")
    return orc.combine(gates, d.reshape(T, k, H), valid.reshape(T, k), acc=acc)
