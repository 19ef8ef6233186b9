"""CPU oracle for the routed-expert hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg may
import this package.  The product library (``mxfp4_routed_expert_k3x_amd``) never does; it
has no CPU fallback.

The arithmetic lives in ``k3x_oracle.c`` (plain C, built with ``-ffp-contract=off`` and
compiled once with a float accumulator -- the verdict oracle -- and once with a double
accumulator -- its self-check).  This module only loads it and marshals numpy arrays.
Every function cites the passage of the kimi-k3-in-c README it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3x_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-Wall", "-Wextra", "-Werror"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (two objects: float and double accumulators)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    objs = []
    for acc, sfx, common in (("float", "f32", True), ("double", "f64", False)):
        obj = os.path.join(_HERE, f"_oracle_{sfx}.o")
        cmd = ["gcc", *_CFLAGS, f"-DORACLE_ACC={acc}", f"-DORACLE_SFX={sfx}", "-c", _SRC, "-o", obj]
        if common:
            cmd.insert(1, "-DORACLE_COMMON=1")
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-shared", "-fopenmp", "-o", tmp, *objs, "-lm"], check=True)
    os.replace(tmp, _LIB)
    for o in objs:
        os.remove(o)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        L.oracle_e2m1.restype = ctypes.c_float
        L.oracle_e2m1.argtypes = [ci]
        L.oracle_e8m0.restype = ctypes.c_float
        L.oracle_e8m0.argtypes = [ci]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16_n.restype = None
        L.oracle_f32_to_bf16_n.argtypes = [P, i64, P]
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ci]
        L.oracle_max_threads.restype = ci
        L.oracle_max_threads.argtypes = []
        L.oracle_sum64.restype = ctypes.c_double
        L.oracle_sum64.argtypes = [P, P, i64]
        L.oracle_route.restype = ci
        L.oracle_route.argtypes = [P, ci, ci, P, P, ci, ci, ci, ctypes.c_float, P, P, P, P]
        L.oracle_rmsnorm_bf16.restype = ci
        L.oracle_rmsnorm_bf16.argtypes = [P, ci, ci, ctypes.c_float, P]
        L.oracle_residual_add_bf16.restype = ci
        L.oracle_residual_add_bf16.argtypes = [P, P, ci, ci]
        L.oracle_rmsnorm_w_f32.restype = ci
        L.oracle_rmsnorm_w_f32.argtypes = [P, ci, ci, P, ctypes.c_float, P]
        L.oracle_mxfp4_matvec_contract.restype = None
        L.oracle_mxfp4_matvec_contract.argtypes = [P, P, P, i64, i64, P]
        L.oracle_expert_forward_contract.restype = ci
        L.oracle_expert_forward_contract.argtypes = [P, i64, i64, P, P, P, P, P, P, ci,
                                                     ctypes.c_float, ctypes.c_float, P, P]
        L.oracle_dense64_bf16.restype = ci
        L.oracle_dense64_bf16.argtypes = [P, P, i64, i64, P]
        L.oracle_glu.restype = ci
        L.oracle_glu.argtypes = [P, P, i64, ci, ctypes.c_float, ctypes.c_float, P]
        for sfx in ("f32", "f64"):
            f = getattr(L, f"oracle_mxfp4_matvec_{sfx}")
            f.restype = None
            f.argtypes = [P, P, P, i64, i64, P]
            f = getattr(L, f"oracle_expert_forward_{sfx}")
            f.restype = None
            f.argtypes = [P, i64, i64, P, P, P, P, P, P, P, P, P, P]
            f = getattr(L, f"oracle_combine_{sfx}")
            f.restype = None
            f.argtypes = [i64, i64, i64, P, P, P, P]
            f = getattr(L, f"oracle_moe_forward_{sfx}")
            f.restype = i64
            f.argtypes = [i64, i64, i64, P, P, P, P, P, P, P, i64, P, P, P, i64, P]
            f = getattr(L, f"oracle_expert_forward_act_{sfx}")
            f.restype = None
            f.argtypes = [P, i64, i64, P, P, P, P, P, P, ci, ctypes.c_float, ctypes.c_float,
                          P, P, P, P]
            f = getattr(L, f"oracle_latent_block_{sfx}")
            f.restype = i64
            f.argtypes = [i64] * 7 + [P, P, P, ci, ctypes.c_float, P, P, P, P, P, P,
                                      ctypes.c_float, P, P, P, P, P, P, ci, ctypes.c_float,
                                      ctypes.c_float, ci, P]
            f = getattr(L, f"oracle_expert_forward_many_{sfx}")
            f.restype = None
            f.argtypes = [P, i64, i64, i64, P, P, P, P, P, P, ci, ctypes.c_float,
                          ctypes.c_float, P]
            f = getattr(L, f"oracle_moe_forward_act_{sfx}")
            f.restype = i64
            f.argtypes = [i64, i64, i64, P, P, P, P, P, P, P, ci, ctypes.c_float, ctypes.c_float,
                          i64, P, P, P, i64, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _sfx(acc):
    assert acc in ("f32", "f64")
    return acc


# --------------------------------------------------------------------------------------
# Thin wrappers
# --------------------------------------------------------------------------------------
def e2m1(code: int) -> float:
    return float(lib().oracle_e2m1(int(code)))


def e8m0(s: int) -> float:
    return float(lib().oracle_e8m0(int(s)))


def bf16_to_f32(bits: int) -> float:
    return float(lib().oracle_bf16_to_f32(int(bits)))


def f32_to_bf16(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(v)))


def bf16_round(a):
    """fp32 array -> bf16 bits, round to nearest even (quiet NaNs kept)."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_n(_p(a), a.size, _p(out))
    return out


def sum64(a, b) -> float:
    a = _c(a, np.float64)
    b = _c(b, np.float64)
    assert a.shape == b.shape and a.size % 8 == 0
    return float(lib().oracle_sum64(_p(a), _p(b), a.size))


def mxfp4_matvec(x, packed, scales, acc="f32"):
    """y = W.x for one MXFP4 matrix; x float32 [K], packed u8 [rows][K/2], scales u8 [rows][K/32]."""
    x = _c(x, np.float32)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = packed.shape
    K = 2 * half
    assert x.shape == (K,) and scales.shape == (rows, K // 32)
    y = np.empty(rows, dtype=np.float32)
    getattr(lib(), f"oracle_mxfp4_matvec_{_sfx(acc)}")(_p(x), _p(packed), _p(scales), rows, K, _p(y))
    return y


ACTIVATIONS = {"swiglu": 0, "situ": 1}


def _act(act):
    """act: "swiglu", or ("situ", b1, b2)."""
    if act == "swiglu" or act is None:
        return 0, 0.0, 0.0
    name, b1, b2 = act
    assert name == "situ"
    return 1, float(b1), float(b2)


def glu(g, u, act=("situ", 4.0, 25.0)):
    """The gated activation in fp32 before the bf16 rounding of h (oracle_glu)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    out = np.empty_like(g)
    a, b1, b2 = _act(act)
    if lib().oracle_glu(_p(g), _p(u), g.size, a, b1, b2, _p(out)) != 0:
        raise ValueError("oracle_glu: bad arguments")
    return out


def expert_forward(x_bf16, ex, acc="f32", want_hidden=False, act="swiglu"):
    """One expert on one activation.  ex has w1_packed..w2_scale (numpy u8).  Returns d
    (float32 [H]) or (h_bf16 [I], g [I], u [I], d [H]).  act: "swiglu" or ("situ", b1, b2)."""
    x = _c(x_bf16, np.uint16)
    H = x.shape[0]
    I = ex.w1_packed.shape[0]
    t = [_c(a, np.uint8) for a in ex.tensors()]
    assert t[0].shape == (I, H // 2) and t[4].shape == (H, I // 2)
    d = np.empty(H, dtype=np.float32)
    h = np.empty(I, dtype=np.uint16) if want_hidden else None
    g = np.empty(I, dtype=np.float32) if want_hidden else None
    u = np.empty(I, dtype=np.float32) if want_hidden else None
    a_, b1, b2 = _act(act)
    getattr(lib(), f"oracle_expert_forward_act_{_sfx(acc)}")(
        _p(x), H, I, *[_p(a) for a in t], a_, b1, b2, _p(h), _p(g), _p(u), _p(d))
    return (h, g, u, d) if want_hidden else d


def expert_forward_many(x_bf16, ex, acc="f32", act="swiglu"):
    """One expert on n activations, expert-major (oracle_expert_forward_many): row t of the
    result equals expert_forward(x_bf16[t], ex) bit for bit.  x bf16 [n][H] -> d fp32 [n][H]."""
    x = _c(x_bf16, np.uint16)
    n, H = x.shape
    I = ex.w1_packed.shape[0]
    t = [_c(a, np.uint8) for a in ex.tensors()]
    assert t[0].shape == (I, H // 2) and t[4].shape == (H, I // 2)
    d = np.empty((n, H), dtype=np.float32)
    a_, b1, b2 = _act(act)
    getattr(lib(), f"oracle_expert_forward_many_{_sfx(acc)}")(
        _p(x), n, H, I, *[_p(a) for a in t], a_, b1, b2, _p(d))
    return d


def combine(gates, d, valid=None, acc="f32"):
    """y[t] = sum_j gates[t][j] * d[t][j] in slot order.  gates [T][k], d [T][k][H]."""
    gates = _c(gates, np.float32)
    d = _c(d, np.float32)
    T, k, H = d.shape
    assert gates.shape == (T, k)
    v = None if valid is None else _c(valid, np.uint8)
    y = np.empty((T, H), dtype=np.float32)
    getattr(lib(), f"oracle_combine_{_sfx(acc)}")(T, k, H, _p(gates), _p(d), _p(v), _p(y))
    return y


def moe_forward(pool, x_bf16, idx, gates, acc="f32", act="swiglu"):
    """Whole forward over a host pool: pool = dict of six u8 arrays [E][rows][cols].
    Returns (y float32 [T][H], drops)."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    idx = _c(idx, np.int32)
    gates = _c(gates, np.float32)
    k = idx.shape[1]
    names = ("w1_packed", "w1_scale", "w3_packed", "w3_scale", "w2_packed", "w2_scale")
    t = [_c(pool[n], np.uint8) for n in names]
    E, I = t[0].shape[0], t[0].shape[1]
    assert t[0].shape == (E, I, H // 2) and t[4].shape == (E, H, I // 2)
    y = np.empty((T, H), dtype=np.float32)
    a_, b1, b2 = _act(act)
    drops = getattr(lib(), f"oracle_moe_forward_act_{_sfx(acc)}")(
        E, H, I, *[_p(a) for a in t], None, a_, b1, b2, T, _p(x), _p(idx), _p(gates), k, _p(y))
    return y, int(drops)


def route(x_bf16, Wr_bf16, bias, topk, renorm=1, routed_scale=1.0, want_scores=False):
    """Sigmoid + correction-bias top-k router.  Returns idx int32 [T][k], gates f32 [T][k]
    (and logits, scores f32 [T][E] when asked)."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    W = _c(Wr_bf16, np.uint16)
    E = W.shape[0]
    assert W.shape == (E, H)
    b = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, topk), dtype=np.int32)
    gates = np.empty((T, topk), dtype=np.float32)
    lg = np.empty((T, E), dtype=np.float32) if want_scores else None
    sc = np.empty((T, E), dtype=np.float32) if want_scores else None
    rc = lib().oracle_route(_p(x), T, H, _p(W), _p(b), E, topk, renorm, routed_scale,
                            _p(idx), _p(gates), _p(lg), _p(sc))
    if rc != 0:
        raise ValueError("oracle_route: bad arguments")
    return (idx, gates, lg, sc) if want_scores else (idx, gates)


def rmsnorm_bf16(x_bf16, eps):
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    out = np.empty_like(x)
    if lib().oracle_rmsnorm_bf16(_p(x), T, H, eps, _p(out)) != 0:
        raise ValueError("oracle_rmsnorm_bf16: bad arguments")
    return out


def residual_add_bf16(x_bf16, y):
    x = _c(x_bf16, np.uint16).copy()
    y = _c(y, np.float32)
    T, H = x.shape
    if lib().oracle_residual_add_bf16(_p(x), _p(y), T, H) != 0:
        raise ValueError("oracle_residual_add_bf16: bad arguments")
    return x


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_max_threads())


def set_threads(n: int) -> None:
    """Sets the threads of the oracle's parallel loops (the results do not depend on it)."""
    lib().oracle_set_threads(int(n))


def rmsnorm_w_f32(x, w, eps):
    """Weighted RMSNorm of fp32 rows -> bf16 bits (w None: weight 1)."""
    x = _c(x, np.float32)
    T, n = x.shape
    out = np.empty((T, n), dtype=np.uint16)
    wp = None if w is None else _c(w, np.float32)
    if lib().oracle_rmsnorm_w_f32(_p(x), T, n, _p(wp), eps, _p(out)) != 0:
        raise ValueError("oracle_rmsnorm_w_f32: bad arguments")
    return out


def mxfp4_matvec_contract(x_f32, packed, scales):
    """The contract's MXFP4 matmul in the listing's order (double, groups in sequence, one
    rounding to float).  x fp32 [K]; packed u8 [rows][K/2]; scales u8 [rows][K/32]."""
    x = _c(x_f32, np.float32)
    p = _c(packed, np.uint8)
    sc = _c(scales, np.uint8)
    rows, K = p.shape[0], x.shape[0]
    assert p.shape == (rows, K // 2) and sc.shape == (rows, K // 32)
    y = np.empty(rows, dtype=np.float32)
    lib().oracle_mxfp4_matvec_contract(_p(x), _p(p), _p(sc), rows, K, _p(y))
    return y


def expert_forward_contract(x_bf16, ex, act="swiglu", want_hidden=False):
    """One expert in the contract's arithmetic (h kept in fp32).  Returns d fp32 [H] (and
    h fp32 [I] with want_hidden)."""
    x = _c(x_bf16, np.uint16)
    H = x.shape[0]
    t = [_c(getattr(ex, n), np.uint8) for n in ("w1_packed", "w1_scale", "w3_packed",
                                                  "w3_scale", "w2_packed", "w2_scale")]
    I = t[0].shape[0]
    a, b1, b2 = _act(act)
    d = np.empty(H, dtype=np.float32)
    h = np.empty(I, dtype=np.float32)
    if lib().oracle_expert_forward_contract(_p(x), H, I, *[_p(v) for v in t], a, b1, b2, _p(h),
                                            _p(d)) != 0:
        raise ValueError("oracle_expert_forward_contract: bad arguments")
    return (d, h) if want_hidden else d


def dense64_bf16(W, v):
    """The contract's bf16 matmul in the fixed 64-way double order: y[r] = (float) sum64(W[r] . v),
    W bf16 [rows][K], v bf16 [K] (K % 8 == 0) -> fp32 [rows]."""
    W = _c(W, np.uint16)
    v = _c(v, np.uint16)
    rows, K = W.shape
    assert v.shape == (K,)
    y = np.empty(rows, dtype=np.float32)
    if lib().oracle_dense64_bf16(_p(W), _p(v), rows, K, _p(y)) != 0:
        raise ValueError("oracle_dense64_bf16: bad arguments")
    return y


def latent_block(x_bf16, Wr, bias, topk, down, up, sh1, sh3, sh2, norm_w, eps, pool,
                 act="swiglu", act_shared=("situ", 4.0, 25.0), renorm=1, routed_scale=1.0,
                 acc="f32"):
    """Stable LatentMoE block for T tokens.  x bf16 [T][D]; Wr bf16 [E][D]; down bf16 [L][D];
    up bf16 [D][L]; sh1, sh3 bf16 [S][D]; sh2 bf16 [D][S]; norm_w fp32 [L] or None; pool the
    routed experts (dense host tensors, hidden = L).  Returns (out fp32 [T][D], drops)."""
    x = _c(x_bf16, np.uint16)
    T, D = x.shape
    Wr = _c(Wr, np.uint16)
    E = Wr.shape[0]
    down, up = _c(down, np.uint16), _c(up, np.uint16)
    sh1, sh3, sh2 = _c(sh1, np.uint16), _c(sh3, np.uint16), _c(sh2, np.uint16)
    L, S = down.shape[0], sh1.shape[0]
    names = ("w1_packed", "w1_scale", "w3_packed", "w3_scale", "w2_packed", "w2_scale")
    t = [_c(pool[n], np.uint8) for n in names]
    I = t[0].shape[1]
    assert down.shape == (L, D) and up.shape == (D, L) and sh2.shape == (D, S)
    assert t[0].shape[2] == L // 2
    b = None if bias is None else _c(bias, np.float32)
    nw = None if norm_w is None else _c(norm_w, np.float32)
    a, b1, b2 = _act(act)
    ash, sb1, sb2 = _act(act_shared)
    if ash == 1 and a == 1:
        assert (sb1, sb2) == (b1, b2), "one pair of caps for routed and shared experts"
    if ash == 1:
        b1, b2 = sb1, sb2
    out = np.empty((T, D), dtype=np.float32)
    drops = getattr(lib(), f"oracle_latent_block_{_sfx(acc)}")(
        T, D, L, I, S, E, topk, _p(x), _p(Wr), _p(b), renorm, routed_scale, _p(down), _p(up),
        _p(sh1), _p(sh3), _p(sh2), _p(nw), eps, *[_p(a_) for a_ in t], a, b1, b2, ash, _p(out))
    if drops < 0:
        raise ValueError("oracle_latent_block: bad arguments")
    return out, int(drops)
