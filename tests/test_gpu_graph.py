"""The layer call captured into a graph, where it forks onto the library's second stream.

A batch of 256 tokens or more with large tiles runs the small tiles' launches on a second stream of
the device, forked from the caller's stream and joined back with events.  Captured into a graph
(after an eager call, which creates that stream), the fork becomes two branches of the graph.
Every replay, with the program's own eager work and synchronizations between the replays, must
give the eager call's results bit for bit."""
import sys

import numpy as np
import pytest

import synth
import quantized_moe_routed_amd as moe
from gpu_util import make_layer, torch_mod, x_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_mod()


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)
    sys.stdout.flush()


def _snapshot(b, T, k):
    return [b.ids.cpu().numpy().copy(), b.w.cpu().numpy().copy(), b.counts.cpu().numpy().copy(),
            b.offsets.cpu().numpy().copy(), b.slot_list.cpu().numpy()[: T * k].copy(), b.y_slot.cpu().numpy().copy(),
            b.out.cpu().numpy().copy()]


def test_graph_replays_equal_the_eager_call(torch):
    from quantized_moe_routed_amd.layer import act_code
    T, H, E, I, k = 300, 128, 4, 128, 2
    _say(f"graph of the forked layer call: T={T} H={H} E={E} I={I} k={k}")
    wl = synth.make(synth.custom(T, H, E, I, k, bias="zipf1.1", gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1,
                                 act="f32", name="graph_t300"))
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    b = layer.buffers(T, act_code(x))
    layer.run(x, b)
    torch.cuda.synchronize()
    counts = b.counts.cpu().numpy()
    lmin = moe.large_tile_min(T)
    assert T >= 256 and counts.max() >= lmin and ((counts > 0) & (counts < lmin)).any()   # both chains run
    ref = _snapshot(b, T, k)

    # other work of the program between replays: a second batch on buffers of its own
    x2 = x.flip(0).contiguous()
    b2 = layer.buffers(T, act_code(x2))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.run(x, b)
    for rep in range(3):
        _say(f"replay {rep}")
        for t in (b.w, b.y_slot, b.out):
            t.fill_(float("nan"))
        for t in (b.ids, b.counts, b.offsets, b.slot_list):
            t.fill_(-7)
        layer.run(x2, b2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(b, T, k)
        for name, a, r in zip(("ids", "w", "counts", "offsets", "slot_list", "y_slot", "out"), got, ref):
            assert np.array_equal(a, r, equal_nan=True), f"replay {rep}: {name} differs from the eager call"
