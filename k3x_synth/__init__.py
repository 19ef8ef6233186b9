"""Seeded synthetic inputs shared by the kernels' tests, the oracle's tests and the bench.

This module holds no arithmetic of the routed-expert method itself: it only makes input
bytes and numbers.  Two kinds of inputs exist:

* Expert weight bytes (MXFP4 nibbles and E8M0 scale bytes).  These are produced by a
  counter-based generator, the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to a per-tensor
  key plus a word counter.  It is implemented twice from that published definition: here
  in numpy (for the experts the oracle needs) and in ``csrc/synth_fill.hip`` (to fill
  the 15.7-189 GB pools directly in device memory).  A GPU test checks they agree.
* Normal and uniform draws (activations, router weights, bias, routing, gates).  These
  are numpy PCG64 draws made on the host and uploaded, so both sides read the same bits.

The tensor shapes follow the Kimi K3 artifact audit, section 4.3 (one routed expert's MXFP4
representation): w1/w3 packed [I][H/2] with scales [I][H/32], w2 packed [H][I/2] with
scales [H][I/32], group 32 along K, low nibble = even element.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------------------
# SplitMix64 (published constants of the generator; see module docstring)
# ---------------------------------------------------------------------------------------
GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# tensor ids inside one expert
W1_PACKED, W1_SCALE, W3_PACKED, W3_SCALE, W2_PACKED, W2_SCALE = range(6)
TENSOR_NAMES = ("w1_packed", "w1_scale", "w3_packed", "w3_scale", "w2_packed", "w2_scale")

# default scale-byte range: integers 118..130 inclusive (13 values)
SCALE_LO = 118
SCALE_COUNT = 13


def fmix64(z):
    """SplitMix64 output step: add the golden gamma, then the two xor-shift-multiply rounds."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z + GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def tensor_key(seed: int, layer: int, expert: int, tensor: int) -> np.uint64:
    """Key of one expert tensor's byte stream."""
    assert 0 <= layer < (1 << 24) and 0 <= expert < (1 << 32) and 0 <= tensor < 256
    h = fmix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF))
    tag = np.uint64((layer << 40) | (expert << 8) | tensor)
    return fmix64(h ^ tag)


def stream_words(key: np.uint64, w0: int, n: int) -> np.ndarray:
    """Words w0..w0+n-1 of the SplitMix64 stream whose state starts at ``key``."""
    i = np.arange(w0, w0 + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return fmix64(key + i * GAMMA)


def packed_bytes(seed, layer, expert, tensor, n_bytes, b0=0):
    """Uniform bytes b0..b0+n_bytes-1 of a packed-nibble tensor (byte b = byte b%8 of word b//8,
    little-endian), so both nibbles are uniform over the 16 E2M1 codes."""
    key = tensor_key(seed, layer, expert, tensor)
    w0 = b0 // 8
    w1 = (b0 + n_bytes + 7) // 8
    words = stream_words(key, w0, w1 - w0)
    raw = words.astype("<u8").view(np.uint8)
    off = b0 - 8 * w0
    return raw[off:off + n_bytes].copy()


def scale_bytes(seed, layer, expert, tensor, n, s0=0, lo=SCALE_LO, count=SCALE_COUNT):
    """Scale bytes s0..s0+n-1: scale s uses the 32-bit half (s % 2) of word s//2 (low half
    first) and maps it to lo + floor(u32 * count / 2^32), i.e. uniform over lo..lo+count-1."""
    key = tensor_key(seed, layer, expert, tensor)
    w0 = s0 // 2
    w1 = (s0 + n + 1) // 2
    words = stream_words(key, w0, w1 - w0)
    halves = np.empty(2 * len(words), dtype=np.uint64)
    halves[0::2] = words & np.uint64(0xFFFFFFFF)
    halves[1::2] = words >> np.uint64(32)
    with np.errstate(over="ignore"):
        v = np.uint64(lo) + ((halves * np.uint64(count)) >> np.uint64(32))
    off = s0 - 2 * w0
    return v[off:off + n].astype(np.uint8)


@dataclass
class ExpertBytes:
    w1_packed: np.ndarray  # u8 [I][H/2]
    w1_scale: np.ndarray   # u8 [I][H/32]
    w3_packed: np.ndarray
    w3_scale: np.ndarray
    w2_packed: np.ndarray  # u8 [H][I/2]
    w2_scale: np.ndarray   # u8 [H][I/32]

    def tensors(self):
        return [getattr(self, n) for n in TENSOR_NAMES]


def tensor_shape(tensor: int, H: int, I: int):
    return {
        W1_PACKED: (I, H // 2), W1_SCALE: (I, H // 32),
        W3_PACKED: (I, H // 2), W3_SCALE: (I, H // 32),
        W2_PACKED: (H, I // 2), W2_SCALE: (H, I // 32),
    }[tensor]


def expert_bytes(seed, layer, expert, H, I, lo=SCALE_LO, count=SCALE_COUNT) -> ExpertBytes:
    """All six tensors of one expert (the C host twin when built, else numpy)."""
    fast = _host_lib()
    out = []
    for t in range(6):
        shp = tensor_shape(t, H, I)
        n = shp[0] * shp[1]
        if fast is not None:
            a = np.empty(n, dtype=np.uint8)
            fast.k3x_synth_host_fill(a.ctypes.data, 0, n, seed & 0xFFFFFFFFFFFFFFFF, layer, expert,
                                     t, t % 2, lo, count)
        elif t % 2 == 0:
            a = packed_bytes(seed, layer, expert, t, n)
        else:
            a = scale_bytes(seed, layer, expert, t, n, lo=lo, count=count)
        out.append(a.reshape(shp))
    return ExpertBytes(*out)


_HOST_SO = None


def _host_lib():
    """ctypes handle of libk3x_synth_host.so (built from csrc/synth_host.c), or None."""
    global _HOST_SO
    if _HOST_SO is None:
        import ctypes
        import os
        here = os.path.dirname(os.path.abspath(__file__))
        so = os.path.join(here, "libk3x_synth_host.so")
        src = os.path.join(here, "csrc", "synth_host.c")
        if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
            try:
                build_host()
            except Exception:
                _HOST_SO = False
                return None
        L = ctypes.CDLL(so)
        L.k3x_synth_host_fill.restype = None
        L.k3x_synth_host_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_int, ctypes.c_uint32,
                                          ctypes.c_uint32]
        _HOST_SO = L
    return _HOST_SO or None


def build_host() -> str:
    import os
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    so = os.path.join(here, "libk3x_synth_host.so")
    tmp = so + ".tmp"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-Werror",
                    os.path.join(here, "csrc", "synth_host.c"), "-o", tmp], check=True)
    os.replace(tmp, so)
    return so


# ---------------------------------------------------------------------------------------
# bf16 bit helpers for input preparation (inputs are stored as bf16 bit patterns)
# ---------------------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + rounding) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(k) & 0xFFFFFFFF for k in key]))


# draw purposes (part of the PCG64 seed key)
P_X, P_WR, P_BIAS, P_ROUTE, P_GATE, P_ZIPF = 1, 2, 3, 4, 5, 6
P_DOWN, P_UP, P_SH1, P_SH3, P_SH2, P_NORMW = 7, 8, 9, 10, 11, 12


def normal_bf16(seed, purpose, layer, shape, std=1.0) -> np.ndarray:
    """N(0, std^2) draws in float64, rounded to float32 then to bf16 (both RNE); bf16 bits."""
    z = _rng(seed, purpose, layer).standard_normal(size=shape) * std
    return f32_to_bf16_bits(z.astype(np.float32))


def normal_f32(seed, purpose, layer, shape, std=1.0) -> np.ndarray:
    z = _rng(seed, purpose, layer).standard_normal(size=shape) * std
    return z.astype(np.float32)


def uniform_routing(seed, T, E, k, layer=0):
    """k distinct experts per token, uniform without replacement; gates U(0,1) in float32
    divided by their float32 sum (summed in slot order)."""
    rng = _rng(seed, P_ROUTE, layer)
    keys = rng.random(size=(T, E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    u = _rng(seed, P_GATE, layer).random(size=(T, k)).astype(np.float32)
    s = np.zeros(T, dtype=np.float32)
    for j in range(k):
        s = (s + u[:, j]).astype(np.float32)
    gates = (u / s[:, None]).astype(np.float32)
    return idx, gates


# Zipf skew of the router bias.  Each expert gets a rank r (a seeded permutation of 1..E);
# bias_e = N(0, 0.01) + ZIPF_ALPHA * (-s * ln r_e).  ZIPF_ALPHA is a fixed constant, chosen
# once offline so that with E = 896, H = 3584, router weights N(0, 0.02) and activations
# N(0, 1), the selection counts of 2048 tokens fall off with popularity rank with a
# log-log slope of about -1.1 over ranks 20..400.  The head cannot follow a power law: an
# expert is picked at most once per token.  The measured slope is reported, not assumed.
ZIPF_S = 1.1
ZIPF_ALPHA = 0.048


def zipf_bias(seed, E, layer=0, std=0.01, s=ZIPF_S, alpha=ZIPF_ALPHA) -> np.ndarray:
    base = normal_f32(seed, P_BIAS, layer, (E,), std).astype(np.float64)
    ranks = _rng(seed, P_ZIPF, layer).permutation(E) + 1
    return (base + alpha * (-s * np.log(ranks))).astype(np.float32)


# ---------------------------------------------------------------------------------------
# The five workloads (sizes of one Kimi K3 MoE layer: H = 3584 latent, I = 3072, top-16)
# ---------------------------------------------------------------------------------------
H_K3 = 3584
I_K3 = 3072
TOPK_K3 = 16


@dataclass(frozen=True)
class Workload:
    name: str
    number: int
    E: int
    T: int
    layers: int
    router: bool
    zipf: bool
    H: int = H_K3
    I: int = I_K3
    topk: int = TOPK_K3

    @property
    def seed(self) -> int:
        return 0x4B335800 + self.number


WORKLOADS = {
    1: Workload("decode_t1_e64", 1, E=64, T=1, layers=1, router=False, zipf=False),
    2: Workload("decode_t1_e896_router", 2, E=896, T=1, layers=1, router=True, zipf=False),
    3: Workload("decode_t32_e896_zipf", 3, E=896, T=32, layers=1, router=True, zipf=True),
    4: Workload("prefill_t4096_e896", 4, E=896, T=4096, layers=1, router=False, zipf=False),
    5: Workload("chain12_t1_e896", 5, E=896, T=1, layers=12, router=True, zipf=True),
}


def expert_bytes_per_expert(H=H_K3, I=I_K3) -> int:
    return 2 * (I * H // 2 + I * H // 32) + (H * I // 2 + H * I // 32)


def router_inputs(w: Workload, layer=0):
    """Router weight bf16 [E][H] ~ N(0, 0.02) and correction bias fp32 [E] ~ N(0, 0.01)
    (Zipf-skewed for the skewed workloads)."""
    Wr = normal_bf16(w.seed, P_WR, layer, (w.E, w.H), std=0.02)
    if w.zipf:
        bias = zipf_bias(w.seed, w.E, layer)
    else:
        bias = normal_f32(w.seed, P_BIAS, layer, (w.E,), std=0.01)
    return Wr, bias


def activations(w: Workload, T=None, layer=0):
    return normal_bf16(w.seed, P_X, layer, (T if T is not None else w.T, w.H), std=1.0)


def log_log_slope(counts, r_lo=20, r_hi=400) -> float:
    """Least-squares slope of log(count) against log(rank), counts sorted descending, over
    ranks r_lo..r_hi that have a non-zero count."""
    c = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    r = np.arange(1, len(c) + 1, dtype=np.float64)
    keep = (c > 0) & (r >= r_lo) & (r <= r_hi)
    c, r = c[keep], r[keep]
    if len(c) < 3:
        return float("nan")
    A = np.vstack([np.log(r), np.ones_like(r)]).T
    slope, _ = np.linalg.lstsq(A, np.log(c), rcond=None)[0]
    return float(slope)



# ---------------------------------------------------------------------------------------
# Device twin (csrc/synth_fill.hip): fills pools directly in GPU memory
# ---------------------------------------------------------------------------------------
import ctypes as _ct
import os as _os

_SYN_DIR = _os.path.dirname(_os.path.abspath(__file__))
SYNTH_LIB = _os.path.join(_SYN_DIR, "libk3x_synth.so")
_synth = None


def build_device() -> str:
    """Compile csrc/synth_fill.hip into libk3x_synth.so (gfx950)."""
    import subprocess
    src = _os.path.join(_SYN_DIR, "csrc", "synth_fill.hip")
    tmp = SYNTH_LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stdout}{r.stderr}")
    _os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def _synth_lib():
    global _synth
    if _synth is None:
        import torch  # noqa: F401  (binds the HIP runtime first)
        if not _os.path.exists(SYNTH_LIB):
            raise ImportError(f"{SYNTH_LIB} missing: call k3x_synth.build_device()")
        L = _ct.CDLL(SYNTH_LIB)
        L.k3x_synth_fill.restype = _ct.c_int
        L.k3x_synth_fill.argtypes = [_ct.c_void_p, _ct.c_uint64, _ct.c_uint32, _ct.c_uint32,
                                     _ct.c_uint64, _ct.c_uint32, _ct.c_uint32, _ct.c_int,
                                     _ct.c_uint32, _ct.c_uint32, _ct.c_void_p]
        _synth = L
    return _synth


def device_fill(t, per_expert: int, e0: int, n_experts: int, seed: int, layer: int, tensor: int,
                lo=SCALE_LO, count=SCALE_COUNT, stream=None):
    """Fill the uint8 device tensor t ([n_experts][per_expert] bytes) with the stream bytes of
    experts e0..e0+n_experts-1 of one tensor id (same bytes as packed_bytes / scale_bytes)."""
    import torch
    kind = 0 if tensor % 2 == 0 else 1
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _synth_lib().k3x_synth_fill(t.data_ptr(), per_expert, e0, n_experts,
                                     seed & 0xFFFFFFFFFFFFFFFF, layer, tensor, kind, lo, count, s)
    if rc != 0:
        raise RuntimeError(f"k3x_synth_fill failed ({rc})")


def device_pool(seed, layer, E, H, I, device="cuda", lo=SCALE_LO, count=SCALE_COUNT):
    """The six expert tensors of one layer, [E][rows][cols] uint8 on the device."""
    import torch
    out = {}
    for t, name in enumerate(TENSOR_NAMES):
        shp = tensor_shape(t, H, I)
        buf = torch.empty((E, shp[0], shp[1]), dtype=torch.uint8, device=device)
        device_fill(buf, shp[0] * shp[1], 0, E, seed, layer, t, lo=lo, count=count)
        out[name] = buf
    return out


def host_pool(seed, layer, E, H, I, experts=None, lo=SCALE_LO, count=SCALE_COUNT):
    """The same bytes on the host (numpy), for the listed experts (default all) stacked in
    that order."""
    ids = range(E) if experts is None else experts
    exps = [expert_bytes(seed, layer, e, H, I, lo=lo, count=count) for e in ids]
    return {n: np.stack([getattr(ex, n) for ex in exps]) for n in TENSOR_NAMES}


# ------------------------------------------------------------------------------------------
# The latent MoE block around the routed experts (kimi-k3-in-c README, Part II section 9):
# full width D, latent L (the routed experts' hidden), routed inter I, S = n_shared * I.
# ------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class LatentShape:
    D: int = 7168
    L: int = H_K3
    I: int = I_K3
    n_shared: int = 2
    E: int = 896
    topk: int = TOPK_K3

    @property
    def S(self) -> int:
        return self.n_shared * self.I


LATENT_K3 = LatentShape()
LATENT_SEED = 0x4B335800 + 6


def latent_inputs(seed, layer, D, L, S, E):
    """Dense bf16 weights of one latent block, each N(0, 1/fan_in) so activations keep unit
    scale: router Wr [E][D] (std 0.02, as the routed workloads), bias N(0, 0.01), down [L][D],
    up [D][L], shared sh1, sh3 [S][D], sh2 [D][S]; the latent RMSNorm weight 1 + N(0, 0.1)."""
    return {
        "Wr": normal_bf16(seed, P_WR, layer, (E, D), std=0.02),
        "bias": normal_f32(seed, P_BIAS, layer, (E,), std=0.01),
        "down": normal_bf16(seed, P_DOWN, layer, (L, D), std=D ** -0.5),
        "up": normal_bf16(seed, P_UP, layer, (D, L), std=L ** -0.5),
        "sh1": normal_bf16(seed, P_SH1, layer, (S, D), std=D ** -0.5),
        "sh3": normal_bf16(seed, P_SH3, layer, (S, D), std=D ** -0.5),
        "sh2": normal_bf16(seed, P_SH2, layer, (D, S), std=S ** -0.5),
        "norm_w": (1.0 + normal_f32(seed, P_NORMW, layer, (L,), std=0.1)).astype(np.float32),
    }
