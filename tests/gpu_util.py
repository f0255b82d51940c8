"""GPU-side test utilities: build a device layer from a workload and run it."""
from __future__ import annotations

import numpy as np

import helpers
import oracle
from helpers import assert_close


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def x_tensor(wl, torch):
    if wl.cfg.act == "bf16":
        return torch.from_numpy(wl.x_bf16.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(wl.x)).cuda()


def make_layer(wl, l2g=None, g2l=None):
    from quantized_moe_routed_amd.layer import MoELayer
    if l2g is None:
        gate, up, down = wl.gate, wl.up, wl.down
    else:
        gate, up, down = wl.gate[l2g], wl.up[l2g], wl.down[l2g]
    return MoELayer(wl.H, wl.I, wl.E, wl.k, wl.cfg.router_fmt, wl.router[0], wl.bias, helpers.fmts(wl),
                    gate, up, down, g2l=g2l)


def run(layer, wl, torch, x=None):
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch) if x is None else x
    b = layer.buffers(wl.T, act_code(x))
    layer.run(x, b)
    torch.cuda.synchronize()
    return dict(ids=b.ids.cpu().numpy(), w=b.w.cpu().numpy(), counts=b.counts.cpu().numpy(),
                offsets=b.offsets.cpu().numpy(), slot_list=b.slot_list.cpu().numpy()[: wl.T * wl.k],
                y=b.y_slot.cpu().numpy(), out=b.out.cpu().numpy())


def check_against_oracle(wl, got, ref, slots_checked=None, what=""):
    T, k = wl.T, wl.k
    tok = ref["tokens"]
    # every token's output, sampled by the oracle or not, is a finite number
    assert np.all(np.isfinite(got["out"])), f"{what}: non-finite outputs"
    assert np.array_equal(got["ids"][tok], ref["ids"]), f"{what}: expert ids differ"
    assert_close(got["w"][tok], ref["w"], f"{what} weights")
    if len(tok) == T:
        counts, offsets, slots = oracle.group(ref["ids"], wl.E)
        assert np.array_equal(got["counts"], counts), f"{what}: counts differ"
        assert np.array_equal(got["offsets"], offsets), f"{what}: offsets differ"
        assert np.array_equal(got["slot_list"], slots), f"{what}: slot_list differs"
    # y rows of the checked tokens' (owned) slots
    rows = np.concatenate([np.arange(t * k, (t + 1) * k) for t in tok])
    ref_y = ref["y"]
    owned = ~np.isnan(ref_y[:, 0])
    if owned.any():
        assert_close(got["y"][rows][owned], ref_y[owned], f"{what} y_slot")
    assert_close(got["out"][tok], ref["out"], f"{what} out")
