"""Python binding of the k3x C ABI (include/k3x.h): argument marshalling only.

Every step of the routed-expert path runs in the HIP kernels of libk3x.so.  There is no CPU
or PyTorch fallback: importing this package without the built library raises.  PyTorch is
used for device memory and streams only.

The functions keep the C names (``k3x_expert_pool_create``, ``k3x_route_topk``,
``k3x_moe_forward``, ...).  Tensors are passed as torch tensors on the GPU; the current torch
stream is used unless a ``stream`` (an integer hipStream_t) is given.
"""
from __future__ import annotations

import ctypes
import os

import torch  # must be imported before libk3x.so so both bind the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3x.so")

K3X_OK = 0
K3X_E_INVALID_ARG = -1
K3X_E_UNSUPPORTED = -2
K3X_E_WORKSPACE = -3
K3X_E_HIP = -4
K3X_E_DROPS = -5


class K3xError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"k3x status {status}: {message}")
        self.status = status


class k3x_pool_desc(ctypes.Structure):
    _fields_ = [
        ("n_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("w1_packed", ctypes.c_void_p),
        ("w1_scale", ctypes.c_void_p),
        ("w3_packed", ctypes.c_void_p),
        ("w3_scale", ctypes.c_void_p),
        ("w2_packed", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p),
        ("stride_bytes", ctypes.c_int64 * 6),
        ("activation", ctypes.c_int32),
        ("situ_b1", ctypes.c_float),
        ("situ_b2", ctypes.c_float),
        ("contract", ctypes.c_int32),
    ]


K3X_ACT_SWIGLU = 0
K3X_ACT_SITU = 1


class k3x_router_desc(ctypes.Structure):
    _fields_ = [
        ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("n_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("renorm", ctypes.c_int32),
        ("routed_scale", ctypes.c_float),
    ]


class k3x_latent_desc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("shared_inter", ctypes.c_int32),
        ("down", ctypes.c_void_p),
        ("up", ctypes.c_void_p),
        ("sh1", ctypes.c_void_p),
        ("sh3", ctypes.c_void_p),
        ("sh2", ctypes.c_void_p),
        ("latent_norm", ctypes.c_int32),
        ("norm_weight", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("shared_activation", ctypes.c_int32),
        ("situ_b1", ctypes.c_float),
        ("situ_b2", ctypes.c_float),
    ]


class k3x_arena_desc(ctypes.Structure):
    _fields_ = [
        ("n_slots", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("host", ctypes.c_void_p * 6),
        ("host_stride", ctypes.c_int64 * 6),
        ("max_slots_per_call", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("situ_b1", ctypes.c_float),
        ("situ_b2", ctypes.c_float),
    ]


K3X_CACHE_LRU, K3X_CACHE_BELADY, K3X_CACHE_PIN_LRU = 0, 1, 2

EXPORTS = (
    "k3x_status_str", "k3x_last_error", "k3x_expert_pool_create", "k3x_expert_pool_destroy",
    "k3x_route_workspace_size", "k3x_route_topk", "k3x_moe_workspace_size", "k3x_moe_forward",
    "k3x_moe_forward_noalloc",
    "k3x_fetch_drops", "k3x_rmsnorm_bf16", "k3x_residual_add_bf16", "k3x_residual_add_rmsnorm_bf16",
    "k3x_latent_workspace_size", "k3x_latent_forward", "k3x_latent_ws_layout",
    "k3x_route_moe_workspace_size", "k3x_route_moe_forward", "k3x_residual_route_moe_forward",
    "k3x_expert_bytes", "k3x_arena_create", "k3x_arena_destroy", "k3x_arena_last_error",
    "k3x_arena_pool", "k3x_arena_getmany", "k3x_arena_pin", "k3x_arena_stats",
    "k3x_arena_moe_forward", "k3x_cache_replay", "k3x_cache_replay_batches",
    "k3x_profiler_create", "k3x_profiler_destroy", "k3x_profiler_attach", "k3x_profiler_reset",
    "k3x_profiler_count", "k3x_profiler_read",
)

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libk3x.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with python -m mxfp4_routed_expert_k3x_amd.build")
    L = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.k3x_status_str.restype = ctypes.c_char_p
    L.k3x_status_str.argtypes = [ctypes.c_int]
    L.k3x_last_error.restype = ctypes.c_char_p
    L.k3x_last_error.argtypes = []
    L.k3x_expert_pool_create.restype = ctypes.c_int
    L.k3x_expert_pool_create.argtypes = [ctypes.POINTER(k3x_pool_desc), ctypes.POINTER(P)]
    L.k3x_expert_pool_destroy.restype = None
    L.k3x_expert_pool_destroy.argtypes = [P]
    L.k3x_route_workspace_size.restype = SZ
    L.k3x_route_workspace_size.argtypes = [ctypes.POINTER(k3x_router_desc), I32]
    L.k3x_route_topk.restype = ctypes.c_int
    L.k3x_route_topk.argtypes = [ctypes.POINTER(k3x_router_desc), P, I32, P, P, P, SZ, P]
    L.k3x_moe_workspace_size.restype = SZ
    L.k3x_moe_workspace_size.argtypes = [P, I32, I32]
    L.k3x_moe_forward.restype = ctypes.c_int
    L.k3x_moe_forward.argtypes = [P, P, I32, P, P, I32, P, P, SZ, P]
    L.k3x_moe_forward_noalloc.restype = ctypes.c_int
    L.k3x_moe_forward_noalloc.argtypes = [P, P, I32, P, P, I32, P, P, P]
    L.k3x_fetch_drops.restype = ctypes.c_int
    L.k3x_fetch_drops.argtypes = [P, ctypes.POINTER(ctypes.c_int64), P]
    L.k3x_rmsnorm_bf16.restype = ctypes.c_int
    L.k3x_rmsnorm_bf16.argtypes = [P, I32, I32, ctypes.c_float, P, P]
    L.k3x_residual_add_bf16.restype = ctypes.c_int
    L.k3x_residual_add_bf16.argtypes = [P, P, I32, I32, P]
    L.k3x_residual_add_rmsnorm_bf16.restype = ctypes.c_int
    L.k3x_residual_add_rmsnorm_bf16.argtypes = [P, P, I32, I32, ctypes.c_float, P, P]
    L.k3x_profiler_create.restype = ctypes.c_int
    LD, RD = ctypes.POINTER(k3x_latent_desc), ctypes.POINTER(k3x_router_desc)
    L.k3x_route_moe_workspace_size.restype = SZ
    L.k3x_route_moe_workspace_size.argtypes = [RD, P, I32]
    L.k3x_route_moe_forward.restype = ctypes.c_int
    L.k3x_route_moe_forward.argtypes = [RD, P, P, I32, P, P, P, P, SZ, P]
    L.k3x_residual_route_moe_forward.restype = ctypes.c_int
    L.k3x_residual_route_moe_forward.argtypes = [RD, P, P, P, ctypes.c_float, P, P, I32, P, P, P,
                                                 P, SZ, P]
    L.k3x_latent_workspace_size.restype = SZ
    L.k3x_latent_workspace_size.argtypes = [LD, P, RD, I32]
    L.k3x_latent_ws_layout.restype = ctypes.c_int
    L.k3x_latent_ws_layout.argtypes = [LD, P, RD, I32, ctypes.POINTER(SZ)]
    L.k3x_latent_forward.restype = ctypes.c_int
    L.k3x_latent_forward.argtypes = [LD, P, RD, P, I32, P, P, SZ, P]
    I64 = ctypes.c_int64
    AD = ctypes.POINTER(k3x_arena_desc)
    L.k3x_expert_bytes.restype = SZ
    L.k3x_expert_bytes.argtypes = [I32, I32]
    L.k3x_arena_create.restype = ctypes.c_int
    L.k3x_arena_create.argtypes = [AD, ctypes.POINTER(P)]
    L.k3x_arena_destroy.restype = None
    L.k3x_arena_destroy.argtypes = [P]
    L.k3x_arena_last_error.restype = ctypes.c_char_p
    L.k3x_arena_last_error.argtypes = []
    L.k3x_arena_pool.restype = P
    L.k3x_arena_pool.argtypes = [P]
    L.k3x_arena_getmany.restype = ctypes.c_int
    L.k3x_arena_getmany.argtypes = [P, I32, P, I32, P, P, P, P]
    L.k3x_arena_pin.restype = ctypes.c_int
    L.k3x_arena_pin.argtypes = [P, I32, I32]
    L.k3x_arena_stats.restype = ctypes.c_int
    L.k3x_arena_stats.argtypes = [P, P, P, P]
    L.k3x_arena_moe_forward.restype = ctypes.c_int
    L.k3x_arena_moe_forward.argtypes = [P, I32, P, I32, P, P, I32, P, P, SZ, P, P, P]
    L.k3x_cache_replay.restype = ctypes.c_int
    L.k3x_cache_replay.argtypes = [P, I64, I32, I32, P, I32, ctypes.POINTER(I64)]
    L.k3x_cache_replay_batches.restype = ctypes.c_int
    L.k3x_cache_replay_batches.argtypes = [P, P, I64, I32, P]
    L.k3x_profiler_create.argtypes = [I32, ctypes.POINTER(P)]
    L.k3x_profiler_destroy.restype = None
    L.k3x_profiler_destroy.argtypes = [P]
    L.k3x_profiler_attach.restype = ctypes.c_int
    L.k3x_profiler_attach.argtypes = [P]
    L.k3x_profiler_reset.restype = ctypes.c_int
    L.k3x_profiler_reset.argtypes = [P]
    L.k3x_profiler_count.restype = I32
    L.k3x_profiler_count.argtypes = [P]
    L.k3x_profiler_read.restype = ctypes.c_int
    L.k3x_profiler_read.argtypes = [P, I32, ctypes.POINTER(ctypes.c_char_p),
                                    ctypes.POINTER(ctypes.c_float)]
    _lib = L
    return L


def lib():
    return load_library()


def _check(st: int):
    if st != K3X_OK:
        L = lib()
        raise K3xError(st, f"{L.k3x_status_str(st).decode()}: {L.k3x_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def k3x_status_str(status: int) -> str:
    return lib().k3x_status_str(status).decode()


def k3x_last_error() -> str:
    return lib().k3x_last_error().decode()


# ------------------------------------------------------------------------------------------
# Expert pool
# ------------------------------------------------------------------------------------------
class Pool:
    """Owns a k3x_pool handle and keeps the borrowed device tensors alive."""

    def __init__(self, handle: int, tensors, E: int, H: int, I: int):
        self.handle = handle
        self.tensors = tensors
        self.E, self.H, self.I = E, H, I

    def close(self):
        if self.handle:
            lib().k3x_expert_pool_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


TENSOR_ORDER = ("w1_packed", "w1_scale", "w3_packed", "w3_scale", "w2_packed", "w2_scale")


def k3x_expert_pool_create(tensors: dict, hidden: int, inter: int, n_experts: int,
                           group: int = 32, strides=None, activation: str = "swiglu",
                           situ_b1: float = 4.0, situ_b2: float = 25.0,
                           contract: bool = False) -> Pool:
    """tensors: the six uint8 device tensors by name (each [E][rows][cols] or any layout that
    matches the strides).  strides: per-expert byte strides (None / 0 = dense).
    activation: "swiglu" or "situ" (SiTU-GLU with caps situ_b1, situ_b2).  contract: the
    floating point contract's arithmetic (double sums in the listing's order, h in fp32; one
    token per call)."""
    d = k3x_pool_desc()
    d.n_experts, d.hidden, d.inter, d.group = n_experts, hidden, inter, group
    d.activation = {"swiglu": K3X_ACT_SWIGLU, "situ": K3X_ACT_SITU}[activation]
    d.situ_b1, d.situ_b2 = situ_b1, situ_b2
    d.contract = 1 if contract else 0
    for name in TENSOR_ORDER:
        t = tensors.get(name)
        setattr(d, name, None if t is None else _ptr(t))
    for k in range(6):
        d.stride_bytes[k] = 0 if strides is None else int(strides[k])
    h = ctypes.c_void_p()
    _check(lib().k3x_expert_pool_create(ctypes.byref(d), ctypes.byref(h)))
    return Pool(h.value, dict(tensors), n_experts, hidden, inter)


def k3x_expert_pool_destroy(pool: Pool):
    pool.close()


# ------------------------------------------------------------------------------------------
# Router
# ------------------------------------------------------------------------------------------
def router_desc(weight, bias, topk, renorm=1, routed_scale=1.0) -> k3x_router_desc:
    """The descriptor holds raw device pointers; it also keeps `weight` and `bias` alive."""
    r = k3x_router_desc()
    r._keep = (weight, bias)
    r.weight = _ptr(weight)
    r.bias = _ptr(bias)
    r.n_experts = int(weight.shape[0])
    r.hidden = int(weight.shape[1])
    r.topk, r.renorm, r.routed_scale = int(topk), int(renorm), float(routed_scale)
    return r


def k3x_route_workspace_size(r: k3x_router_desc, T: int) -> int:
    return int(lib().k3x_route_workspace_size(ctypes.byref(r), int(T)))


def k3x_route_topk(r: k3x_router_desc, x, T: int, idx_out, gates_out, ws, ws_bytes=None,
                   stream=None):
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().k3x_route_topk(ctypes.byref(r), _ptr(x), int(T), _ptr(idx_out),
                                _ptr(gates_out), _ptr(ws), int(nbytes), _stream(stream)))


# ------------------------------------------------------------------------------------------
# Expert forward
# ------------------------------------------------------------------------------------------
def k3x_moe_workspace_size(pool: Pool, T: int, topk: int) -> int:
    return int(lib().k3x_moe_workspace_size(pool.handle, int(T), int(topk)))


def k3x_moe_forward(pool: Pool, x, T: int, idx, gates, topk: int, y, ws, ws_bytes=None,
                    stream=None):
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().k3x_moe_forward(pool.handle, _ptr(x), int(T), _ptr(idx), _ptr(gates),
                                 int(topk), _ptr(y), _ptr(ws), int(nbytes), _stream(stream)))


def k3x_route_moe_workspace_size(r: k3x_router_desc, pool: Pool, T: int) -> int:
    return int(lib().k3x_route_moe_workspace_size(ctypes.byref(r), pool.handle, int(T)))


def k3x_route_moe_forward(r: k3x_router_desc, pool: Pool, x, T: int, idx_out, gates_out, y, ws,
                          ws_bytes=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().k3x_route_moe_forward(ctypes.byref(r), pool.handle, _ptr(x), int(T),
                                       _ptr(idx_out), _ptr(gates_out), _ptr(y), _ptr(ws),
                                       int(nbytes), _stream(stream)))


def k3x_residual_route_moe_forward(r: k3x_router_desc, pool: Pool, x, y_prev, eps: float, x_next,
                                   xn, T: int, idx_out, gates_out, y, ws, ws_bytes=None,
                                   stream=None):
    """y_prev and x_next may be None (the first layer: RMSNorm of x alone)."""
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().k3x_residual_route_moe_forward(
        ctypes.byref(r), pool.handle, _ptr(x), _ptr(y_prev), float(eps), _ptr(x_next), _ptr(xn),
        int(T), _ptr(idx_out), _ptr(gates_out), _ptr(y), _ptr(ws), int(nbytes),
        _stream(stream)))


K3X_NOALLOC_SCRATCH_BYTES = 32 << 20


def k3x_moe_forward_noalloc(pool: Pool, x, T: int, idx, gates, topk: int, y, drops_out=None,
                            stream=None):
    """k3x_moe_forward with the library's built-in scratch as its workspace (allocates
    nothing); drops_out: None or a device int64 tensor of one element."""
    _check(lib().k3x_moe_forward_noalloc(pool.handle, _ptr(x), int(T), _ptr(idx), _ptr(gates),
                                         int(topk), _ptr(y), _ptr(drops_out), _stream(stream)))


def k3x_fetch_drops(ws, stream=None) -> int:
    n = ctypes.c_int64(0)
    st = lib().k3x_fetch_drops(_ptr(ws), ctypes.byref(n), _stream(stream))
    if st not in (K3X_OK, K3X_E_DROPS):
        _check(st)
    return int(n.value)


def k3x_rmsnorm_bf16(x, T: int, H: int, eps: float, out, stream=None):
    _check(lib().k3x_rmsnorm_bf16(_ptr(x), int(T), int(H), float(eps), _ptr(out), _stream(stream)))


def k3x_residual_add_bf16(x, y, T: int, H: int, stream=None):
    _check(lib().k3x_residual_add_bf16(_ptr(x), _ptr(y), int(T), int(H), _stream(stream)))


def k3x_residual_add_rmsnorm_bf16(x, y, T: int, H: int, eps: float, out, stream=None):
    _check(lib().k3x_residual_add_rmsnorm_bf16(_ptr(x), _ptr(y), int(T), int(H), float(eps),
                                               _ptr(out), _stream(stream)))


# ------------------------------------------------------------------------------------------
# Latent MoE block
# ------------------------------------------------------------------------------------------
def latent_desc(down, up, sh1, sh3, sh2, norm_weight=None, eps=1e-5, latent_norm=1,
                shared_activation="situ", situ_b1=4.0, situ_b2=25.0) -> k3x_latent_desc:
    """down bf16 [L][D], up [D][L], sh1/sh3 [S][D], sh2 [D][S] (device tensors of bf16 bits);
    norm_weight fp32 [L] or None (weight 1)."""
    d = k3x_latent_desc()
    d.hidden, d.shared_inter = int(down.shape[1]), int(sh1.shape[0])
    d.down, d.up, d.sh1, d.sh3, d.sh2 = (_ptr(t) for t in (down, up, sh1, sh3, sh2))
    d.latent_norm = int(latent_norm)
    d.norm_weight = _ptr(norm_weight)
    d.eps = float(eps)
    d.shared_activation = {"swiglu": K3X_ACT_SWIGLU, "situ": K3X_ACT_SITU}[shared_activation]
    d.situ_b1, d.situ_b2 = float(situ_b1), float(situ_b2)
    return d


def k3x_latent_workspace_size(d: k3x_latent_desc, pool: Pool, r: k3x_router_desc, T: int) -> int:
    return int(lib().k3x_latent_workspace_size(ctypes.byref(d), pool.handle, ctypes.byref(r),
                                               int(T)))


LATENT_WS_FIELDS = ("idx", "gates", "z", "acc", "s", "moe")


def k3x_latent_ws_layout(d: k3x_latent_desc, pool: Pool, r: k3x_router_desc, T: int) -> dict:
    """{name: byte offset} of the block's intermediates in its workspace."""
    offs = (ctypes.c_size_t * 6)()
    _check(lib().k3x_latent_ws_layout(ctypes.byref(d), pool.handle, ctypes.byref(r), int(T), offs))
    return dict(zip(LATENT_WS_FIELDS, (int(v) for v in offs)))


def k3x_latent_forward(d: k3x_latent_desc, pool: Pool, r: k3x_router_desc, x, T: int, out, ws,
                       ws_bytes=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(lib().k3x_latent_forward(ctypes.byref(d), pool.handle, ctypes.byref(r), _ptr(x),
                                    int(T), _ptr(out), _ptr(ws), int(nbytes), _stream(stream)))


# ------------------------------------------------------------------------------------------
# Expert arena (pools larger than HBM) and trace replay
# ------------------------------------------------------------------------------------------
class Arena:
    """Owns a k3x_arena handle; keeps the borrowed pinned backing tensors alive.  .pool is a
    Pool view of the slots (owned by the arena)."""

    def __init__(self, handle, backing, n_slots, H, I):
        self.handle = handle
        self.backing = backing
        self.pool = Pool(0, {}, n_slots, H, I)
        self.pool.handle = lib().k3x_arena_pool(handle)
        self.pool.close = lambda: None  # the arena owns it

    def close(self):
        if self.handle:
            lib().k3x_arena_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def k3x_expert_bytes(hidden: int, inter: int) -> int:
    return int(lib().k3x_expert_bytes(int(hidden), int(inter)))


def k3x_arena_create(host: dict, n_slots: int, n_layers: int, n_experts: int, hidden: int,
                     inter: int, max_slots_per_call: int = 1024, host_strides=None,
                     activation: str = "swiglu", situ_b1: float = 4.0, situ_b2: float = 25.0,
                     group: int = 32) -> Arena:
    """host: the six pinned host tensors (or integer addresses) by name, expert (l, e) at
    index l * n_experts + e of each (stride = host_strides[k] bytes, None = dense)."""
    d = k3x_arena_desc()
    d.n_slots, d.n_layers, d.n_experts = n_slots, n_layers, n_experts
    d.hidden, d.inter, d.group = hidden, inter, group
    for k, name in enumerate(TENSOR_ORDER):
        d.host[k] = _ptr(host[name])
        d.host_stride[k] = 0 if host_strides is None else int(host_strides[k])
    d.max_slots_per_call = max_slots_per_call
    d.activation = {"swiglu": K3X_ACT_SWIGLU, "situ": K3X_ACT_SITU}[activation]
    d.situ_b1, d.situ_b2 = situ_b1, situ_b2
    h = ctypes.c_void_p()
    st = lib().k3x_arena_create(ctypes.byref(d), ctypes.byref(h))
    if st != K3X_OK:
        raise K3xError(st, f"{k3x_status_str(st)}: {lib().k3x_arena_last_error().decode()} "
                           f"{k3x_last_error()}")
    return Arena(h.value, dict(host), n_slots, hidden, inter)


def k3x_arena_destroy(arena: Arena):
    arena.close()


def k3x_arena_last_error() -> str:
    return lib().k3x_arena_last_error().decode()


def k3x_arena_pool(arena: Arena) -> Pool:
    return arena.pool


def k3x_arena_getmany(arena: Arena, layer: int, experts, stream=None):
    """experts: host int sequence.  Returns (slots list, hits, misses)."""
    import numpy as np
    e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    out = np.empty(len(e), dtype=np.int32)
    h, m = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().k3x_arena_getmany(arena.handle, int(layer), e.ctypes.data, len(e),
                                   out.ctypes.data, ctypes.byref(h), ctypes.byref(m),
                                   _stream(stream)))
    return out.tolist(), h.value, m.value


def k3x_arena_pin(arena: Arena, layer: int, expert: int):
    _check(lib().k3x_arena_pin(arena.handle, int(layer), int(expert)))


def k3x_arena_stats(arena: Arena):
    h, m, b = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().k3x_arena_stats(arena.handle, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)))
    return h.value, m.value, b.value


def k3x_arena_moe_forward(arena: Arena, layer: int, x, T: int, idx, gates, topk: int, y, ws,
                          ws_bytes=None, stream=None):
    """Returns (hits, misses) of the call."""
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    h, m = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().k3x_arena_moe_forward(arena.handle, int(layer), _ptr(x), int(T), _ptr(idx),
                                       _ptr(gates), int(topk), _ptr(y), _ptr(ws), int(nbytes),
                                       ctypes.byref(h), ctypes.byref(m), _stream(stream)))
    return h.value, m.value


def k3x_cache_replay(trace, cap: int, policy: int = K3X_CACHE_LRU, pinned=()) -> int:
    import numpy as np
    t = np.ascontiguousarray(np.asarray(trace, dtype=np.int64))
    p = np.ascontiguousarray(np.asarray(list(pinned), dtype=np.int64))
    hits = ctypes.c_int64(0)
    _check(lib().k3x_cache_replay(t.ctypes.data, len(t), int(cap), int(policy),
                                  p.ctypes.data if len(p) else None, len(p), ctypes.byref(hits)))
    return hits.value


def k3x_cache_replay_batches(batches, cap: int):
    """batches: list of key lists.  Returns the slot given to every key, batch by batch."""
    import numpy as np
    keys = np.ascontiguousarray(np.asarray([k for b in batches for k in b], dtype=np.int64))
    starts = np.ascontiguousarray(np.cumsum([0] + [len(b) for b in batches]).astype(np.int64))
    out = np.empty(len(keys), dtype=np.int32)
    _check(lib().k3x_cache_replay_batches(keys.ctypes.data, starts.ctypes.data, len(batches),
                                          int(cap), out.ctypes.data))
    res, j = [], 0
    for b in batches:
        res.append(out[j:j + len(b)].tolist())
        j += len(b)
    return res


# ------------------------------------------------------------------------------------------
# Conveniences over the C calls (allocation of outputs and workspaces with torch)
# ------------------------------------------------------------------------------------------
def alloc_workspace(nbytes: int, device="cuda"):
    """A 256-byte aligned uint8 device buffer (torch's caching allocator aligns to 512)."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def moe_forward(pool: Pool, x, idx, gates, y=None, ws=None, stream=None):
    """y = k3x_moe_forward(...) with y and workspace allocated on demand.  x: bf16 [T][H]
    (a torch.bfloat16 or int16/uint16 tensor of bf16 bits)."""
    T, topk = int(idx.shape[0]), int(idx.shape[1])
    if y is None:
        y = torch.empty((T, pool.H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = alloc_workspace(k3x_moe_workspace_size(pool, T, topk), x.device)
    k3x_moe_forward(pool, x, T, idx, gates, topk, y, ws, stream=stream)
    return y, ws


def route_topk(weight, bias, x, topk, renorm=1, routed_scale=1.0, idx=None, gates=None,
               ws=None, stream=None):
    T = int(x.shape[0])
    r = router_desc(weight, bias, topk, renorm, routed_scale)
    if idx is None:
        idx = torch.empty((T, topk), dtype=torch.int32, device=x.device)
    if gates is None:
        gates = torch.empty((T, topk), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = alloc_workspace(k3x_route_workspace_size(r, T), x.device)
    k3x_route_topk(r, x, T, idx, gates, ws, stream=stream)
    return idx, gates, ws


# ------------------------------------------------------------------------------------------
# Kernel timing (HIP events around every kernel the library launches from this thread)
# ------------------------------------------------------------------------------------------
def k3x_profiler_create(capacity: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().k3x_profiler_create(int(capacity), ctypes.byref(h)))
    return h.value


def k3x_profiler_destroy(prof: int):
    lib().k3x_profiler_destroy(prof)


def k3x_profiler_attach(prof):
    _check(lib().k3x_profiler_attach(prof))


def k3x_profiler_reset(prof: int):
    _check(lib().k3x_profiler_reset(prof))


def k3x_profiler_count(prof: int) -> int:
    return int(lib().k3x_profiler_count(prof))


def k3x_profiler_read(prof: int, i: int):
    """(kernel name, milliseconds) of recorded launch i."""
    name = ctypes.c_char_p()
    ms = ctypes.c_float()
    _check(lib().k3x_profiler_read(prof, int(i), ctypes.byref(name), ctypes.byref(ms)))
    return name.value.decode(), float(ms.value)


def profiler_durations(prof: int):
    """{kernel name: [ms, ...]} of everything recorded since the last reset."""
    out = {}
    for i in range(k3x_profiler_count(prof)):
        n, ms = k3x_profiler_read(prof, i)
        out.setdefault(n, []).append(ms)
    return out
