"""Device-resident weights and buffers for one routed-expert layer (or one
owned share of it), and the four library calls that run it.

The weights arrive in the definition layout (array of blocks); they are
re-laid into the planar device layout by the library's host packer and copied
to device memory once.  ``run`` issues moe_route, moe_group_tokens,
moe_expert_forward and moe_combine on one stream with no host sync.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import (ACT_BF16, ACT_F32, W_F32, Experts, combine, expert_forward, group_tokens, layer_forward,
               layer_forward_noalloc, pack_planar,
               plan_check,
               qmat, route, route_table, shared_expert_forward, shared_expert_workspace, table_check,
               workspace_size)


def _to_dev(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceMatrix:
    """A stack of n planar matrices on the device."""

    def __init__(self, fmt: int, aos: np.ndarray, n: int, rows: int, cols: int, device):
        codes, scales = pack_planar(fmt, aos, n, rows, cols)
        self.fmt, self.n, self.rows, self.cols = fmt, n, rows, cols
        self.codes = _to_dev(codes, device)
        self.scales = _to_dev(scales, device)

    def qmat(self):
        return qmat(self.fmt, self.rows, self.cols, self.codes, self.scales)

    def nbytes(self) -> int:
        return self.codes.numel() + (0 if self.scales is None else self.scales.numel())


@dataclass
class Buffers:
    T: int
    xt: int
    ids: torch.Tensor
    w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    slot_list: torch.Tensor
    y_slot: torch.Tensor
    out: torch.Tensor
    route_ws: torch.Tensor          # views into ws: the router's part, then the experts' part
    fwd_ws: torch.Tensor
    ws: torch.Tensor


class MoELayer:
    """One layer's router plus an owned expert stack on one device.

    gate/up/down are definition-layout stacks [E_local, rows, row_bytes] of the
    OWNED experts in local-id order; g2l maps global ids to local ids (-1 =
    unowned) or is None when every expert is owned with local = global."""

    def __init__(self, H: int, I: int, E: int, k: int, router_fmt: int, router_aos: np.ndarray,
                 bias: Optional[np.ndarray], fmts, gate_aos, up_aos, down_aos, g2l: Optional[np.ndarray] = None,
                 device=None):
        self.device = torch.device(device or "cuda")
        self.H, self.I, self.E, self.k = H, I, E, k
        self.E_local = gate_aos.shape[0]
        if g2l is not None:
            plan_check(g2l, self.E_local)
        self.router = DeviceMatrix(router_fmt, router_aos, 1, E, H, self.device)
        self.bias = _to_dev(None if bias is None else np.asarray(bias, np.float32), self.device)
        self.gate = DeviceMatrix(fmts[0], gate_aos, self.E_local, I, H, self.device)
        self.up = DeviceMatrix(fmts[1], up_aos, self.E_local, I, H, self.device)
        self.down = DeviceMatrix(fmts[2], down_aos, self.E_local, H, I, self.device)
        self.g2l = _to_dev(None if g2l is None else np.asarray(g2l, np.int32), self.device)
        self._router_q = self.router.qmat()
        self._experts = Experts(self.gate.qmat(), self.up.qmat(), self.down.qmat(), self.E_local)

    def expert_bytes(self) -> int:
        return self.gate.nbytes() + self.up.nbytes() + self.down.nbytes()

    def buffers(self, T: int, xt: int) -> Buffers:
        d = self.device
        rws, _, fws = workspace_size(T, self.H, self.I, self.k, self.E, self.E_local, xt)
        i32 = dict(dtype=torch.int32, device=d)
        ws = torch.empty(rws + max(fws, 1), dtype=torch.uint8, device=d)
        return Buffers(
            T=T, xt=xt,
            ids=torch.empty((T, self.k), **i32),
            w=torch.empty((T, self.k), dtype=torch.float32, device=d),
            counts=torch.empty(self.E, **i32),
            offsets=torch.empty(self.E + 1, **i32),
            slot_list=torch.empty(max(T * self.k, 1), **i32),
            y_slot=torch.zeros((T * self.k, self.H), dtype=torch.float32, device=d),
            out=torch.empty((T, self.H), dtype=torch.float32, device=d),
            route_ws=ws[:rws] if rws else ws[:1],
            fwd_ws=ws[rws:],
            ws=ws,
        )

    # the four calls, each a thin wrapper
    def route(self, x: torch.Tensor, b: Buffers, stream=None):
        route(x, b.xt, b.T, self.H, self._router_q, self.bias, self.k, b.ids, b.w, b.route_ws,
              b.route_ws.numel(), stream)

    def route_table(self, x: torch.Tensor, b: Buffers, token_ids: torch.Tensor, table: torch.Tensor, stream=None):
        """Table routing: token t takes the experts of row token_ids[t] of table [V, k] (device)."""
        route_table(x, b.xt, b.T, self.H, self._router_q, self.bias, token_ids, table, table.shape[0], self.k, b.ids,
                    b.w, b.route_ws, b.route_ws.numel(), stream)

    def group(self, b: Buffers, stream=None):
        group_tokens(b.ids, b.T, self.k, self.E, b.counts, b.offsets, b.slot_list, None, 0, stream)

    def forward(self, x: torch.Tensor, b: Buffers, stream=None):
        expert_forward(x, b.xt, b.T, self.H, self.I, self.k, self._experts, self.g2l, self.E, self.E_local,
                       b.counts, b.offsets, b.slot_list, b.y_slot, b.fwd_ws, b.fwd_ws.numel(), stream)

    def combine(self, b: Buffers, stream=None):
        combine(b.y_slot, b.w, b.ids, self.g2l, b.T, self.k, self.H, self.E, b.out, stream)

    def run_calls(self, x: torch.Tensor, b: Buffers, stream=None):
        """The layer as the four calls in turn."""
        self.route(x, b, stream)
        self.group(b, stream)
        self.forward(x, b, stream)
        self.combine(b, stream)
        return b.out

    def run_table(self, x: torch.Tensor, b: Buffers, token_ids: torch.Tensor, table: torch.Tensor, stream=None):
        """The layer with table routing: route_table, then the grouping, experts and combine calls."""
        self.route_table(x, b, token_ids, table, stream)
        self.group(b, stream)
        self.forward(x, b, stream)
        self.combine(b, stream)
        return b.out

    def run(self, x: torch.Tensor, b: Buffers, stream=None):
        """The layer as one call (moe_layer_forward): the four calls' results, fewer launches."""
        layer_forward(x, b.xt, b.T, self.H, self.I, self.k, self._router_q, self.bias, self._experts, self.g2l,
                      self.E, self.E_local, b.ids, b.w, b.counts, b.offsets, b.slot_list, b.y_slot, b.out, b.ws,
                      b.ws.numel(), stream)
        return b.out


    def run_noalloc(self, x: torch.Tensor, b: Buffers, stream=None):
        """The layer as one call on the library's own scratch (moe_layer_forward_noalloc): b's
        workspace is not used; results equal run's bit for bit."""
        layer_forward_noalloc(x, b.xt, b.T, self.H, self.I, self.k, self._router_q, self.bias, self._experts,
                              self.g2l, self.E, self.E_local, b.ids, b.w, b.counts, b.offsets, b.slot_list, b.y_slot,
                              b.out, stream)
        return b.out


def act_code(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return ACT_F32
    if x.dtype == torch.bfloat16:
        return ACT_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


__all__ = ["MoELayer", "DeviceMatrix", "Buffers", "act_code", "W_F32"]


class SharedExpert:
    """The shared expert beside the routed ones: one expert stack (gate/up I x H, down H x I) on one
    device; add_to(x, out) adds its output to the routed output out in place."""

    def __init__(self, H: int, I: int, fmt: int, gate_aos, up_aos, down_aos, device=None):
        self.device = torch.device(device or "cuda")
        self.H, self.I = H, I
        self.gate = DeviceMatrix(fmt, gate_aos, 1, I, H, self.device)
        self.up = DeviceMatrix(fmt, up_aos, 1, I, H, self.device)
        self.down = DeviceMatrix(fmt, down_aos, 1, H, I, self.device)
        self._experts = Experts(self.gate.qmat(), self.up.qmat(), self.down.qmat(), 1)
        self._ws = {}   # one workspace per stream handle

    def nbytes(self) -> int:
        return self.gate.nbytes() + self.up.nbytes() + self.down.nbytes()

    def add_to(self, x: torch.Tensor, out: torch.Tensor, stream=None):
        """out += the shared expert of x, on `stream` (a torch stream or a raw handle; None: the
        current stream).  Each stream gets its own workspace, recorded on that stream, so a regrown
        workspace is not handed out again while the stream's earlier calls may still use it."""
        T, xt = x.shape[0], act_code(x)
        n = shared_expert_workspace(T, self.H, self.I, xt)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        elif isinstance(stream, int):
            stream = torch.cuda.ExternalStream(stream, device=self.device)
        key = stream.cuda_stream
        ws = self._ws.get(key)
        if ws is None or ws.numel() < n:
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)
            ws.record_stream(stream)
            self._ws[key] = ws
        shared_expert_forward(x, xt, T, self.H, self.I, self._experts, out, ws, ws.numel(), stream)
        return out
