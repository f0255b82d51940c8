"""Seeded synthetic workloads for the routed-expert MoE layer.

This package only makes inputs: it draws the activations, router and expert
weights, biases and placement histograms of the five workloads below, and
encodes drawn weights into the block formats the layer reads.  It holds none
of the layer's arithmetic; the CPU oracle (``oracle/``) and the GPU library
(``quantized_moe_routed_amd``) both consume what it returns and import nothing
from each other.

Workloads (shapes of a DeepSeek-V4-class routed-expert layer):

====  =====  ====  ===  ====  ==  =====================  ======  ==========================
cfg   T      H     E    I     k   gate / up / down       router  other
====  =====  ====  ===  ====  ==  =====================  ======  ==========================
1     4      256   8    128   2   Q8_0 / Q8_0 / Q8_0     fp32    tiny, CPU-seconds scale
2     1      4096  256  2048  8   Q2SM / Q2SM / Q2SM     Q8_0    single-token decode
3     32     4096  256  2048  8   Q2SM / Q2SM / Q8_0     Q8_0    bias N(0, 0.5)
4     2048   4096  256  2048  8   Q2SM / Q2SM / Q8_0     Q8_0    Zipf(1.1) bias, bf16 x
5     128    4096  256  2048  8   Q2SM / Q2SM / Q8_0     Q8_0    LPT share of 128 experts
====  =====  ====  ===  ====  ==  =====================  ======  ==========================

All weights are N(0, 0.02) before encoding, activations N(0, 1).  Workloads
3-5 share their weight draws; workload 2 encodes the same gate/up draws and
encodes its down draws as Q2SM.  Token t of every workload is the same draw,
so a longer token list extends a shorter one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
# MOE_SYNTH_LIB names another build of the same source (the sanitizer test builds one with
# -fsanitize=address,undefined); it is loaded as it is, without building
_LIB_OVERRIDE = os.environ.get("MOE_SYNTH_LIB")
_LIB_PATH = _LIB_OVERRIDE or os.path.join(_HERE, "libsynth.so")
_lib = None
_lock = threading.Lock()

FMT_F32, FMT_Q8_0, FMT_Q2SM = 0, 1, 2
FMT_NAMES = {FMT_F32: "f32", FMT_Q8_0: "q8_0", FMT_Q2SM: "q2sm"}
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q2SM: 12}

# stream roles (stream id = role << 20 | index)
_X, _ROUTER, _BIAS, _ZIPF, _HIST, _PPERM, _GATE, _UP, _DOWN = 1, 2, 3, 4, 5, 6, 16, 17, 18
_TABLE, _TOKID = 7, 8
_SGATE, _SUP, _SDOWN = 19, 20, 21
W_SIGMA = 0.02


def build(force: bool = False) -> str:
    if _LIB_OVERRIDE:
        return _LIB_PATH
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_double, ctypes.c_void_p)
            L.synth_normal_f32.argtypes = [u64, u64, i64, dbl, vp]
            L.synth_u64.argtypes = [u64, u64, i64, vp]
            L.synth_permutation.argtypes = [u64, u64, i32, vp]
            L.synth_quant_matrices.argtypes = [u64, u64, i32, i32, i32, dbl, i32, vp]
            L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
            L.synth_f32_to_f16.argtypes = [vp, i64, vp]
            L.synth_f32_to_f16_bits.argtypes = [ctypes.c_float]
            L.synth_f32_to_f16_bits.restype = ctypes.c_uint16
            _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def normal(seed: int, stream: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, n, sigma, _ptr(out))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, stream, n, _ptr(out))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_f16(_ptr(a), a.size, _ptr(out))
    return out


def row_bytes(fmt: int, cols: int) -> int:
    return cols * 4 if fmt == FMT_F32 else (cols // 32) * BLOCK_BYTES[fmt]


def quant_matrices(seed: int, stream0: int, n_mat: int, rows: int, cols: int, fmt: int,
                   sigma: float = W_SIGMA) -> np.ndarray:
    """n_mat drawn matrices [rows, cols], encoded; returns uint8 [n_mat, rows, row_bytes]."""
    assert cols % 32 == 0 and cols <= 16384
    out = np.empty((n_mat, rows, row_bytes(fmt, cols)), dtype=np.uint8)
    lib().synth_quant_matrices(seed, stream0, n_mat, rows, cols, sigma, fmt, _ptr(out))
    return out


@dataclass
class Config:
    cfg: int
    name: str
    T: int
    H: int
    E: int
    I: int
    k: int
    gate_fmt: int
    up_fmt: int
    down_fmt: int
    router_fmt: int
    act: str                 # "f32" or "bf16"
    bias: Optional[str]      # None, "normal0.5", "zipf1.1"
    share: bool = False      # expert-parallel share workload


CONFIGS = {
    1: Config(1, "tiny", 4, 256, 8, 128, 2, FMT_Q8_0, FMT_Q8_0, FMT_Q8_0, FMT_F32, "f32", None),
    2: Config(2, "decode", 1, 4096, 256, 2048, 8, FMT_Q2SM, FMT_Q2SM, FMT_Q2SM, FMT_Q8_0, "f32", None),
    3: Config(3, "batched_decode", 32, 4096, 256, 2048, 8, FMT_Q2SM, FMT_Q2SM, FMT_Q8_0, FMT_Q8_0,
              "f32", "normal0.5"),
    4: Config(4, "prefill", 2048, 4096, 256, 2048, 8, FMT_Q2SM, FMT_Q2SM, FMT_Q8_0, FMT_Q8_0,
              "bf16", "zipf1.1"),
    5: Config(5, "ep_share", 128, 4096, 256, 2048, 8, FMT_Q2SM, FMT_Q2SM, FMT_Q8_0, FMT_Q8_0,
              "f32", None, share=True),
}


@dataclass
class Workload:
    cfg: Config
    T: int
    x: np.ndarray                     # fp32 [T, H]: the layer input's values (bf16 inputs upcast exactly)
    x_bf16: Optional[np.ndarray]      # uint16 [T, H] bf16 bits when act == "bf16"
    router: np.ndarray                # uint8 [1, E, row_bytes] in router_fmt (fp32 rows as raw bytes)
    bias: Optional[np.ndarray]        # fp32 [E]
    gate: Optional[np.ndarray]        # uint8 [E, I, row_bytes(H)]
    up: Optional[np.ndarray]          # uint8 [E, I, row_bytes(H)]
    down: Optional[np.ndarray]        # uint8 [E, H, row_bytes(I)]
    load_hist: Optional[np.ndarray] = None   # int64 [E]: expert-load histogram for placement
    local_perm: Optional[np.ndarray] = None  # int32 [E]: seeded order for a permuted local numbering
    extra: dict = field(default_factory=dict)

    @property
    def H(self): return self.cfg.H

    @property
    def E(self): return self.cfg.E

    @property
    def I(self): return self.cfg.I

    @property
    def k(self): return self.cfg.k


_weight_cache: dict = {}


def _matrices(seed: int, role: int, n: int, rows: int, cols: int, fmt: int) -> np.ndarray:
    key = (seed, role, n, rows, cols, fmt)
    if key not in _weight_cache:
        if len(_weight_cache) >= 8:  # a full weight set is a few GB: keep a handful at most
            _weight_cache.pop(next(iter(_weight_cache)))
        _weight_cache[key] = quant_matrices(seed, role << 20, n, rows, cols, fmt)
    return _weight_cache[key]


def _weights(cfg: Config, seed: int):
    router = _matrices(seed, _ROUTER, 1, cfg.E, cfg.H, cfg.router_fmt)
    gate = _matrices(seed, _GATE, cfg.E, cfg.I, cfg.H, cfg.gate_fmt)
    up = _matrices(seed, _UP, cfg.E, cfg.I, cfg.H, cfg.up_fmt)
    down = _matrices(seed, _DOWN, cfg.E, cfg.H, cfg.I, cfg.down_fmt)
    return router, gate, up, down


def shared_expert(seed: int, H: int, I: int, fmt: int = FMT_Q8_0):
    """One shared expert (gate, up [1, I, row bytes of H], down [1, H, row bytes of I]) drawn as
    the routed experts are, N(0, 0.02), in one format (Q8_0 by default)."""
    return (_matrices(seed, _SGATE, 1, I, H, fmt), _matrices(seed, _SUP, 1, I, H, fmt),
            _matrices(seed, _SDOWN, 1, H, I, fmt))


def route_table(seed: int, V: int, E: int, k: int) -> np.ndarray:
    """A token-id routing table [V, k] int32: row v holds k distinct experts, the first k of a
    seeded permutation of 0..E-1 drawn for that row (a stand-in for a tokenizer's table)."""
    return np.stack([permutation(seed, (_TABLE << 20) + v, E)[:k] for v in range(V)]).astype(np.int32)


def token_ids(seed: int, T: int, V: int, first: int = 0) -> np.ndarray:
    """Token ids of tokens first .. first+T-1, uniform over 0..V-1 (a seeded permutation's
    entries, taken modulo V)."""
    n = first + T
    return (permutation(seed, _TOKID << 20, max(n, V))[first:n] % V).astype(np.int32)


def tokens(seed: int, T: int, H: int, first: int = 0) -> np.ndarray:
    """fp32 activations for tokens first .. first+T-1, N(0, 1)."""
    n = (first + T) * H
    return normal(seed, _X << 20, n, 1.0)[first * H:].reshape(T, H)


def custom(T: int, H: int, E: int, I: int, k: int, gate_fmt: int = FMT_Q8_0, up_fmt: int = FMT_Q8_0,
           down_fmt: int = FMT_Q8_0, router_fmt: int = FMT_Q8_0, act: str = "f32",
           bias: Optional[str] = None, share: bool = False, name: str = "custom") -> Config:
    """A workload shape other than the five above (small parity cases, edge cases)."""
    return Config(0, name, T, H, E, I, k, gate_fmt, up_fmt, down_fmt, router_fmt, act, bias, share)


def make(cfg_id, seed: int = 0, T: Optional[int] = None, first_token: int = 0,
         experts: bool = True) -> Workload:
    """Build workload cfg_id (1..5, or a Config from custom()).  T overrides the
    token count (a prefix of the token stream); experts=False skips drawing the
    expert weights (gate/up/down are then None)."""
    cfg = cfg_id if isinstance(cfg_id, Config) else CONFIGS[cfg_id]
    T = cfg.T if T is None else T
    if experts:
        router, gate, up, down = _weights(cfg, seed)
    else:
        router = _matrices(seed, _ROUTER, 1, cfg.E, cfg.H, cfg.router_fmt)
        gate = up = down = None
    x = tokens(seed, T, cfg.H, first_token)
    x_bf16 = None
    if cfg.act == "bf16":
        x_bf16 = f32_to_bf16_bits(x)
        x = bf16_bits_to_f32(x_bf16).reshape(T, cfg.H)
    bias = None
    if cfg.bias == "normal0.5":
        bias = normal(seed, _BIAS << 20, cfg.E, 0.5)
    elif cfg.bias == "zipf1.1":
        # popularity rank 1 + perm[e]; bias -s * ln(rank) makes selection odds Zipf-like
        rank = permutation(seed, _ZIPF << 20, cfg.E).astype(np.float64) + 1.0
        bias = (-1.1 * np.log(rank)).astype(np.float32)
    wl = Workload(cfg, T, x, x_bf16, router, bias, gate, up, down)
    if cfg.share:
        g = normal(seed, _HIST << 20, cfg.E, 1.0).astype(np.float64)
        wl.load_hist = np.rint(64.0 * np.exp(0.75 * g)).astype(np.int64)
        wl.local_perm = permutation(seed, _PPERM << 20, cfg.E)
    return wl
