"""moe_layer_forward_noalloc (the layer call on the library's own per-device scratch array, for
callers that cannot allocate) against moe_layer_forward with a caller workspace: the same ids,
weights, grouping, y_slot and output bit for bit, and the output within the oracle's tolerance, on
two calls in a row whose second batch is smaller (the scratch keeps the first call's contents)."""
import sys

import numpy as np
import pytest

import synth
import quantized_moe_routed_amd as moe
from helpers import oracle_expect
from gpu_util import check_against_oracle, make_layer, torch_mod, x_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    return torch_mod()


def _outputs(b, T, k):
    return dict(ids=b.ids.cpu().numpy(), w=b.w.cpu().numpy(), counts=b.counts.cpu().numpy(),
                offsets=b.offsets.cpu().numpy(), slot_list=b.slot_list.cpu().numpy()[: T * k],
                y=b.y_slot.cpu().numpy(), out=b.out.cpu().numpy())


def _both(layer, wl, torch):
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    res = []
    for noalloc in (False, True):
        b = layer.buffers(wl.T, act_code(x))
        b.out.fill_(float("nan"))
        (layer.run_noalloc if noalloc else layer.run)(x, b)
        torch.cuda.synchronize()
        res.append(_outputs(b, wl.T, wl.k))
    return res


@pytest.mark.parametrize("cfg,T1,T2", [(3, 32, 5), (2, 8, 1), (4, 96, 40)])
def test_noalloc_equals_layer_call_twice(torch, cfg, T1, T2):
    for T in (T1, T2):
        _say(f"noalloc vs layer call: cfg{cfg} T={T}")
        wl = synth.make(cfg, T=T)
        layer = make_layer(wl)
        ref, got = _both(layer, wl, torch)
        for name in ref:
            assert np.array_equal(ref[name].view(np.uint8), got[name].view(np.uint8)), f"{name} differs, T={T}"
        tok = list(range(0, T, max(1, T // 8)))
        check_against_oracle(wl, got, oracle_expect(wl, tokens=tok), what=f"noalloc cfg{cfg} T={T}")


def test_noalloc_large_tiles_first(torch):
    """A batch of 300 tokens with large tiles at small shapes (it fits the scratch array): the call
    without allocation runs first (in a fresh process no second stream exists yet, and this call
    does not create one), then the layer call; both give the same results bit for bit."""
    from quantized_moe_routed_amd.layer import act_code
    T = 300
    _say(f"noalloc with large tiles first: T={T}")
    wl = synth.make(synth.custom(T, 128, 4, 128, 2, bias="zipf1.1", gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1,
                                 act="f32", name="noalloc_t300"))
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    res = []
    for noalloc in (True, False):
        b = layer.buffers(T, act_code(x))
        b.out.fill_(float("nan"))
        (layer.run_noalloc if noalloc else layer.run)(x, b)
        torch.cuda.synchronize()
        res.append(_outputs(b, T, wl.k))
    got, ref = res
    counts = got["counts"]
    lmin = moe.large_tile_min(T)
    assert counts.max() >= lmin and ((counts > 0) & (counts < lmin)).any()   # both tile kinds
    for name in ref:
        assert np.array_equal(ref[name].view(np.uint8), got[name].view(np.uint8)), f"{name} differs"


def test_noalloc_share_and_refusal(torch):
    """An owned share (g2l table) gives the layer call's partial bit for bit; a batch whose workspace
    exceeds the scratch array is refused before anything runs, and its outputs stay untouched."""
    _say("noalloc share and refusal")
    wl = synth.make(5, T=24)
    owner = moe.place_lpt(wl.load_hist, 2)
    g2l, l2g = moe.share_tables(owner, 0)
    layer = make_layer(wl, l2g=l2g, g2l=g2l)
    ref, got = _both(layer, wl, torch)
    for name in ref:
        assert np.array_equal(ref[name].view(np.uint8), got[name].view(np.uint8)), f"{name} differs (share)"
    big = synth.make(4, T=512)
    layer = make_layer(big)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(big, torch)
    b = layer.buffers(512, act_code(x))
    b.out.fill_(-7.0)
    with pytest.raises(moe.MoeError) as e:
        layer.run_noalloc(x, b)
    assert e.value.status == moe.ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((b.out == -7.0).all())
