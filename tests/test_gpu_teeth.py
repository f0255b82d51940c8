"""Test strength on the GPU path (aeonmindai/arc PR #89, "The tests are the teeth").

The page applies three mutations to an expert-parallel implementation and
shows which equivalence tests catch each: dropping the global-to-local remap,
never masking unowned slots, and combining with unmasked weights.  Here the
same three breaks are applied to the inputs of the C ABI, with no kernel
changed, and the invariants this suite relies on must catch every one:

* a share's partial plus its complement's partial equals the full layer;
* a share's partial equals the one computed under the correct tables.

Each mutation runs next to its unmutated control, which must pass.  The
shares hold many experts with local id != global id, so a wrong remap cannot
be right by coincidence (the page's one-expert-per-share blind spot).
A last test checks that rows of unowned slots are left untouched."""
import sys

import numpy as np
import pytest

import synth
import quantized_moe_routed_amd as moe
from helpers import close_report, MAX_ABS_FRAC, REL_L2
from gpu_util import make_layer, torch_mod, x_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-teeth] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    return torch_mod()


def _within(got, ref):
    mabs, mref, rel = close_report(got, ref)
    return mabs <= MAX_ABS_FRAC * mref and rel <= REL_L2


def _setup(T=24):
    wl = synth.make(5, T=T)
    owner = moe.place_lpt(wl.load_hist, 2)
    tabs = [moe.share_tables(owner, sh) for sh in (0, 1)]
    for g2l, l2g in tabs:
        assert len(l2g) >= 2 and np.any(l2g != np.arange(len(l2g)))
    return wl, tabs


def _partial(layer, wl, torch, x, g2l_dev=None, combine_g2l="layer", y_slot=None):
    """One share's partial through the four calls; g2l_dev replaces the layer's device table for the
    expert call (a mutation that the host check at load would refuse), combine_g2l the table the
    combine call gets ("layer": the layer's own, None: no table), y_slot a buffer to reuse."""
    from quantized_moe_routed_amd.layer import act_code
    b = layer.buffers(wl.T, act_code(x))
    if y_slot is not None:
        b.y_slot = y_slot
    layer.route(x, b)
    layer.group(b)
    table = layer.g2l if g2l_dev is None else g2l_dev
    moe.expert_forward(x, b.xt, b.T, layer.H, layer.I, layer.k, layer._experts, table, layer.E, layer.E_local,
                       b.counts, b.offsets, b.slot_list, b.y_slot, b.fwd_ws, b.fwd_ws.numel())
    cg = layer.g2l if combine_g2l == "layer" else combine_g2l
    moe.combine(b.y_slot, b.w, b.ids, cg, b.T, layer.k, layer.H, layer.E, b.out)
    torch.cuda.synchronize()
    return b.out.cpu().numpy().astype(np.float64), b


def test_dropped_remap_is_caught(torch):
    """Mutation 1: the owned experts' local ids rotated by one (still a valid bijection, so the host
    check at load passes it): each owned slot runs a neighbouring expert's weights."""
    _say("mutation: dropped remap")
    wl, tabs = _setup()
    x = x_tensor(wl, torch)
    full, _ = _partial(make_layer(wl), wl, torch, x)
    layers = [make_layer(wl, l2g=l2g, g2l=g2l) for g2l, l2g in tabs]
    a, _ = _partial(layers[0], wl, torch, x)
    b, _ = _partial(layers[1], wl, torch, x)
    assert _within(a + b, full), "control: A + B must equal the full layer"
    g2l, l2g = tabs[0]
    rot = np.where(g2l >= 0, (g2l + 1) % len(l2g), -1).astype(np.int32)
    moe.plan_check(rot, len(l2g))   # the break passes the load-time check
    a_bad, _ = _partial(layers[0], wl, torch, x, g2l_dev=torch.from_numpy(rot).cuda())
    assert not _within(a_bad + b, full), "A + B = full did not catch a dropped remap"
    assert not np.array_equal(a_bad, a), "the partial did not change under a dropped remap"


def test_unmasked_slots_are_caught(torch):
    """Mutation 2: unowned experts mapped to local expert 0 instead of -1, so no slot is masked (the
    host check at load refuses this table, so it is swapped in on the device after loading)."""
    _say("mutation: never mask")
    wl, tabs = _setup()
    x = x_tensor(wl, torch)
    full, _ = _partial(make_layer(wl), wl, torch, x)
    layers = [make_layer(wl, l2g=l2g, g2l=g2l) for g2l, l2g in tabs]
    b, _ = _partial(layers[1], wl, torch, x)
    g2l, l2g = tabs[0]
    nomask = np.where(g2l >= 0, g2l, 0).astype(np.int32)
    with pytest.raises(moe.MoeError):
        moe.plan_check(nomask, len(l2g))
    dev = torch.from_numpy(nomask).cuda()
    a_bad, _ = _partial(layers[0], wl, torch, x, g2l_dev=dev, combine_g2l=dev)
    assert not _within(a_bad + b, full), "A + B = full did not catch unmasked slots"


def test_unmasked_combine_is_caught(torch):
    """Mutation 3: both shares write one reused y_slot buffer (A, then B), and A's combine is given
    no owner table, so it keeps the weights of B's slots."""
    _say("mutation: combine with unmasked weights")
    wl, tabs = _setup()
    x = x_tensor(wl, torch)
    full, _ = _partial(make_layer(wl), wl, torch, x)
    layers = [make_layer(wl, l2g=l2g, g2l=g2l) for g2l, l2g in tabs]
    shared_y = torch.zeros((wl.T * wl.k, wl.H), dtype=torch.float32, device="cuda")
    a, ba = _partial(layers[0], wl, torch, x, y_slot=shared_y)
    b, _ = _partial(layers[1], wl, torch, x, y_slot=shared_y)
    assert _within(a + b, full), "control: masked combines add up to the full layer"
    # A's combine again, now over the buffer that also holds B's rows, without A's owner table
    moe.combine(shared_y, ba.w, ba.ids, None, wl.T, wl.k, wl.H, wl.E, ba.out)
    torch.cuda.synchronize()
    a_bad = ba.out.cpu().numpy().astype(np.float64)
    assert not _within(a_bad + b, full), "A + B = full did not catch a combine with unmasked weights"


@pytest.mark.parametrize("T", [24, 300])
def test_unowned_rows_are_left_untouched(torch, T):
    """y_slot filled with a NaN sentinel before a share's layer call: every row of an unowned slot
    still holds the sentinel bit for bit, every owned row is finite (T=300: large tiles too)."""
    _say(f"sentinel rows T={T}")
    if T == 24:
        wl, tabs = _setup(T)
    else:
        wl = synth.make(synth.custom(T, 256, 16, 128, 2, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1,
                                     bias="zipf1.1", name="sentinel_large"))
        owner = moe.place_lpt(np.arange(16, dtype=np.int64) + 1, 2)
        tabs = [moe.share_tables(owner, sh) for sh in (0, 1)]
    g2l, l2g = tabs[0]
    layer = make_layer(wl, l2g=l2g, g2l=g2l)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    b = layer.buffers(T, act_code(x))
    sentinel = np.int32(0x7FC0BEEF)
    b.y_slot.view(torch.int32).fill_(int(sentinel))
    layer.run(x, b)
    torch.cuda.synchronize()
    ids = b.ids.cpu().numpy().reshape(-1)
    owned = g2l[ids] >= 0
    y = b.y_slot.cpu().numpy()
    if T == 300:
        assert b.counts.cpu().numpy()[l2g].max() >= moe.large_tile_min(T)
    assert owned.any() and (~owned).any()
    assert np.all(y[~owned].view(np.int32) == sentinel), "an unowned slot's row was written"
    assert np.all(np.isfinite(y[owned])), "an owned slot's row was not written"
