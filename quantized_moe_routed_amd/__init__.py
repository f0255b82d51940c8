"""Python binding of libmoe.so, the gfx950 routed-expert MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The
functions keep the C names of ``include/moe.h`` (without the ``moe_`` prefix)
and raise :class:`MoeError` on a non-zero status.  If the library has not
been built, importing this package fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

# PyTorch ships its own HIP runtime (same soname as ROCm's).  Loading torch
# first makes libmoe bind to that one runtime; loading libmoe first would put
# a second HIP runtime in the process, which then finds no device.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_DEVICE, ERR_WORKSPACE, ERR_HIP = range(6)
W_F32, W_Q8_0, W_Q2SM = 0, 1, 2
ACT_F32, ACT_BF16 = 0, 1


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class QMat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat), ("n_experts", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(python quantized_moe_routed_amd/build.py); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    i32, sz, vp, psz = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_version.restype = ctypes.c_char_p
    L.moe_large_tile_min.argtypes = [i32]
    L.moe_large_tile_min.restype = ctypes.c_int32
    L.moe_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, psz, psz, psz]
    L.moe_route.argtypes = [vp, i32, i32, i32, ctypes.POINTER(QMat), vp, i32, vp, vp, vp, sz, vp]
    L.moe_route_table.argtypes = [vp, i32, i32, i32, ctypes.POINTER(QMat), vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    L.moe_table_check.argtypes = [vp, i32, i32, i32]
    L.moe_shared_expert_workspace.argtypes = [i32, i32, i32, i32, psz]
    L.moe_shared_expert_forward.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(Experts), vp, vp, sz, vp]
    L.moe_group_tokens.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.moe_expert_forward.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(Experts), vp, i32, i32,
                                     vp, vp, vp, vp, vp, sz, vp]
    L.moe_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]
    L.moe_layer_forward.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(QMat), vp, ctypes.POINTER(Experts), vp,
                                    i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_layer_forward_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(QMat), vp,
                                            ctypes.POINTER(Experts), vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_planar_bytes.argtypes = [i32, i32, i32, psz, psz]
    L.moe_pack_planar.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    L.moe_place_lpt.argtypes = [vp, i32, i32, vp]
    L.moe_share_tables.argtypes = [vp, i32, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_int32)]
    L.moe_plan_check.argtypes = [vp, i32, i32]
    L.moe_trace_kernel.argtypes = [ctypes.c_char_p, vp, vp, i32, ctypes.POINTER(ctypes.c_int32)]
    L.moe_trace_kernel_every.argtypes = [ctypes.c_char_p, vp, vp, i32, i32, ctypes.POINTER(ctypes.c_int32)]
    for f in ("moe_trace_kernel", "moe_trace_kernel_every", "moe_workspace_size", "moe_route", "moe_group_tokens", "moe_expert_forward", "moe_combine",
              "moe_layer_forward", "moe_layer_forward_noalloc", "moe_route_table", "moe_table_check",
              "moe_shared_expert_workspace", "moe_shared_expert_forward",
              "moe_planar_bytes", "moe_pack_planar", "moe_place_lpt", "moe_share_tables", "moe_plan_check"):
        getattr(L, f).restype = ctypes.c_int
    return L


lib = _load()

EXPORTS = ("moe_last_error", "moe_version", "moe_large_tile_min", "moe_workspace_size", "moe_route", "moe_group_tokens",
           "moe_expert_forward", "moe_combine", "moe_layer_forward", "moe_planar_bytes", "moe_pack_planar", "moe_place_lpt",
           "moe_share_tables", "moe_plan_check", "moe_trace_kernel", "moe_trace_kernel_every", "moe_route_table",
           "moe_table_check", "moe_shared_expert_workspace", "moe_shared_expert_forward", "moe_layer_forward_noalloc")


def last_error() -> str:
    return lib.moe_last_error().decode()


def version() -> str:
    return lib.moe_version().decode()


def _check(status: int):
    if status != OK:
        raise MoeError(status, last_error())


def _ptr(t) -> Optional[int]:
    """Device or host address of a torch tensor / numpy array (None stays NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def qmat(fmt: int, rows: int, cols: int, codes, scales) -> QMat:
    return QMat(fmt, rows, cols, _ptr(codes), _ptr(scales))


def large_tile_min(T: int) -> int:
    """Fewest slots of one expert that go to 128-slot tiles in a batch of T tokens (0: none)."""
    return int(lib.moe_large_tile_min(T))


# ---------------------------------------------------------------- device calls
def workspace_size(T, H, I, k, E, E_local, xt):
    r, g, f = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.moe_workspace_size(T, H, I, k, E, E_local, xt, ctypes.byref(r), ctypes.byref(g), ctypes.byref(f)))
    return r.value, g.value, f.value


def route(x, xt, T, H, router: QMat, bias, k, ids, w, ws, ws_bytes, stream=None):
    _check(lib.moe_route(_ptr(x), xt, T, H, ctypes.byref(router), _ptr(bias), k, _ptr(ids), _ptr(w),
                         _ptr(ws), ws_bytes, _stream(stream)))


def group_tokens(ids, T, k, E, counts, offsets, slot_list, ws=None, ws_bytes=0, stream=None):
    _check(lib.moe_group_tokens(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(slot_list), _ptr(ws),
                                ws_bytes, _stream(stream)))


def expert_forward(x, xt, T, H, I, k, local: Experts, g2l, E, E_local, counts, offsets, slot_list, y_slot,
                   ws, ws_bytes, stream=None):
    _check(lib.moe_expert_forward(_ptr(x), xt, T, H, I, k, ctypes.byref(local), _ptr(g2l), E, E_local,
                                  _ptr(counts), _ptr(offsets), _ptr(slot_list), _ptr(y_slot), _ptr(ws), ws_bytes,
                                  _stream(stream)))


def combine(y_slot, w, ids, g2l, T, k, H, E, out, stream=None):
    _check(lib.moe_combine(_ptr(y_slot), _ptr(w), _ptr(ids), _ptr(g2l), T, k, H, E, _ptr(out), _stream(stream)))


def layer_forward(x, xt, T, H, I, k, router: QMat, bias, local: Experts, g2l, E, E_local, ids, w, counts, offsets,
                  slot_list, y_slot, out, ws, ws_bytes, stream=None):
    _check(lib.moe_layer_forward(_ptr(x), xt, T, H, I, k, ctypes.byref(router), _ptr(bias), ctypes.byref(local),
                                 _ptr(g2l), E, E_local, _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets),
                                 _ptr(slot_list), _ptr(y_slot), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def layer_forward_noalloc(x, xt, T, H, I, k, router: QMat, bias, local: Experts, g2l, E, E_local, ids, w, counts,
                          offsets, slot_list, y_slot, out, stream=None):
    """moe_layer_forward on the library's own per-device scratch array: no workspace argument."""
    _check(lib.moe_layer_forward_noalloc(_ptr(x), xt, T, H, I, k, ctypes.byref(router), _ptr(bias),
                                         ctypes.byref(local), _ptr(g2l), E, E_local, _ptr(ids), _ptr(w), _ptr(counts),
                                         _ptr(offsets), _ptr(slot_list), _ptr(y_slot), _ptr(out), _stream(stream)))


# ---------------------------------------------------------------- host helpers
def planar_bytes(fmt, rows, cols):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.moe_planar_bytes(fmt, rows, cols, ctypes.byref(c), ctypes.byref(s)))
    return c.value, s.value


def pack_planar(fmt: int, aos: np.ndarray, n: int, rows: int, cols: int):
    """Definition-layout bytes of n matrices -> (codes, scales) numpy planes."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8)
    cb, sb = planar_bytes(fmt, rows, cols)
    codes = np.empty(n * cb, dtype=np.uint8)
    scales = np.empty(max(n * sb, 1), dtype=np.uint8)
    _check(lib.moe_pack_planar(fmt, n, rows, cols, _ptr(aos), _ptr(codes), _ptr(scales)))
    return codes, (scales if sb else None)


def place_lpt(load: np.ndarray, n_shares: int) -> np.ndarray:
    load = np.ascontiguousarray(load, dtype=np.int64)
    owner = np.empty(len(load), dtype=np.int32)
    _check(lib.moe_place_lpt(_ptr(load), len(load), n_shares, _ptr(owner)))
    return owner


def share_tables(owner: np.ndarray, share: int, local_order: Optional[np.ndarray] = None):
    owner = np.ascontiguousarray(owner, dtype=np.int32)
    E = len(owner)
    g2l = np.empty(E, dtype=np.int32)
    l2g = np.empty(E, dtype=np.int32)
    n = ctypes.c_int32()
    lo = None if local_order is None else np.ascontiguousarray(local_order, dtype=np.int32)
    _check(lib.moe_share_tables(_ptr(owner), E, share, _ptr(lo), _ptr(g2l), _ptr(l2g), ctypes.byref(n)))
    return g2l, l2g[:n.value].copy()


class KernelTrace:
    """Live per-kernel timing: HIP events around launches 0, every, 2 every, ... of one kernel
    (at most n of them).

    with KernelTrace("ffn_gateup", n) as tr: ...launches...; then tr.times_ms()"""

    def __init__(self, name: str, n: int, every: int = 1):
        import torch
        self.name = name.encode()
        self.n = n
        self.every = every
        self._ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self._ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self._ev0 + self._ev1:
            e.record()          # materialise the underlying hipEvent_t
        torch.cuda.synchronize()
        self._h0 = (ctypes.c_void_p * n)(*[e.cuda_event for e in self._ev0])
        self._h1 = (ctypes.c_void_p * n)(*[e.cuda_event for e in self._ev1])
        self.count = ctypes.c_int32(0)

    def __enter__(self):
        _check(lib.moe_trace_kernel_every(self.name, self._h0, self._h1, self.n, self.every,
                                          ctypes.byref(self.count)))
        return self

    def __exit__(self, *exc):
        lib.moe_trace_kernel(None, None, None, 0, None)

    def times_ms(self):
        import torch
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(self._ev0[: self.count.value], self._ev1[: self.count.value])]


def route_table(x, xt, T, H, router: QMat, bias, token_ids, table, V, k, ids, w, ws, ws_bytes, stream=None):
    _check(lib.moe_route_table(_ptr(x), xt, T, H, ctypes.byref(router), _ptr(bias), _ptr(token_ids), _ptr(table), V,
                               k, _ptr(ids), _ptr(w), _ptr(ws), ws_bytes, _stream(stream)))


def shared_expert_workspace(T, H, I, xt) -> int:
    n = ctypes.c_size_t()
    _check(lib.moe_shared_expert_workspace(T, H, I, xt, ctypes.byref(n)))
    return n.value


def shared_expert_forward(x, xt, T, H, I, shared: Experts, out, ws, ws_bytes, stream=None):
    _check(lib.moe_shared_expert_forward(_ptr(x), xt, T, H, I, ctypes.byref(shared), _ptr(out), _ptr(ws), ws_bytes,
                                         _stream(stream)))


def table_check(table: np.ndarray, E: int):
    table = np.ascontiguousarray(table, dtype=np.int32)
    V, k = table.shape
    _check(lib.moe_table_check(_ptr(table), V, k, E))


def plan_check(g2l: np.ndarray, E_local: int):
    g2l = np.ascontiguousarray(g2l, dtype=np.int32)
    _check(lib.moe_plan_check(_ptr(g2l), len(g2l), E_local))
