"""The single-token layer call (the decode step), beyond the configs' own parity cases.

In the layer call, the gate/up launch of a single token selects the experts itself, and its
workgroup (0, 0) stores the routing results. This file checks that path:

* against the oracle, over several tokens: 2-bit and Q8_0 formats, fp32 and bf16 activations,
  and small or odd shapes (few tiles, k = E, an odd number of blocks per row, k = 1);
* bit for bit against the four separate calls (route, group, expert forward, combine): ids,
  weights, grouping, the y rows of owned slots, and the output;
* expert-parallel shares at T=1: each share's partial equals the four calls' partial bit for
  bit, the two partials add up to the full layer, and a share that owns none of the token's
  experts gives exactly zero;
* consecutive calls on one set of buffers: every call equals a call on fresh buffers bit for
  bit."""
import sys

import numpy as np
import pytest

import synth
import quantized_moe_routed_amd as moe
from helpers import assert_close, oracle_expect
from gpu_util import check_against_oracle, make_layer, torch_mod, x_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-single-token] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    return torch_mod()


def _result(b, torch):
    torch.cuda.synchronize()
    return dict(ids=b.ids.cpu().numpy(), w=b.w.cpu().numpy(), counts=b.counts.cpu().numpy(),
                offsets=b.offsets.cpu().numpy(), slot_list=b.slot_list.cpu().numpy()[: b.T * b.ids.shape[1]],
                y=b.y_slot.cpu().numpy(), out=b.out.cpu().numpy())


def _layer_call(layer, x, torch, b=None):
    from quantized_moe_routed_amd.layer import act_code
    b = layer.buffers(1, act_code(x)) if b is None else b
    layer.run(x, b)
    return _result(b, torch)


def _four_calls(layer, x, torch):
    from quantized_moe_routed_amd.layer import act_code
    b = layer.buffers(1, act_code(x))
    layer.run_calls(x, b)
    return _result(b, torch)


def _same_as_calls(got, ref, owned_rows, what):
    for key in ("ids", "w", "counts", "offsets", "slot_list"):
        assert got[key].tobytes() == ref[key].tobytes(), f"{what}: {key} differs from the four calls"
    assert got["y"][owned_rows].tobytes() == ref["y"][owned_rows].tobytes(), f"{what}: y rows differ"
    assert got["out"].tobytes() == ref["out"].tobytes(), f"{what}: out differs from the four calls"


def _owned_rows(got, g2l=None):
    ids = got["ids"].reshape(-1)
    return np.arange(len(ids)) if g2l is None else np.flatnonzero(g2l[ids] >= 0)


@pytest.mark.parametrize("first", [0, 1, 7, 23])
def test_decode_tokens_against_oracle_and_calls(torch, first):
    """The decode shapes (E=256, k=8, 2-bit experts, fp32): token `first` of the stream."""
    _say(f"decode token {first}")
    wl = synth.make(2, T=1, first_token=first)
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    got = _layer_call(layer, x, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what=f"decode token {first}")
    _same_as_calls(got, _four_calls(layer, x, torch), _owned_rows(got), f"decode token {first}")


@pytest.mark.parametrize("fmts,act", [((1, 1, 1), "f32"), ((2, 2, 1), "bf16"), ((1, 1, 2), "f32"), ((2, 2, 2), "bf16")])
def test_formats_and_activations(torch, fmts, act):
    """Every pairing of gate/up and down formats, and bf16 activations (no lo plane), at H=1024,
    I=512, E=64, k=6."""
    _say(f"formats {fmts} {act}")
    cfg = synth.custom(1, 1024, 64, 512, 6, gate_fmt=fmts[0], up_fmt=fmts[1], down_fmt=fmts[2], router_fmt=1,
                       act=act, bias="normal0.5", name="single_token_fmts")
    wl = synth.make(cfg)
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    got = _layer_call(layer, x, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what=f"{fmts} {act}")
    _same_as_calls(got, _four_calls(layer, x, torch), _owned_rows(got), f"{fmts} {act}")


@pytest.mark.parametrize("H,I,E,k", [(256, 128, 8, 2), (160, 96, 8, 8), (2080, 224, 16, 3), (4096, 2048, 256, 1)])
def test_small_and_odd_shapes(torch, H, I, E, k):
    """Few tiles, k = E, an odd number of blocks per row, and k = 1."""
    _say(f"shape H={H} I={I} E={E} k={k}")
    cfg = synth.custom(1, H, E, I, k, gate_fmt=2, up_fmt=2, down_fmt=2, router_fmt=1,
                       bias="normal0.5", name="single_token_shapes")
    wl = synth.make(cfg)
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    got = _layer_call(layer, x, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what=f"H={H} I={I} E={E} k={k}")
    _same_as_calls(got, _four_calls(layer, x, torch), _owned_rows(got), f"H={H} k={k}")


def test_shares_at_one_token(torch):
    """Expert-parallel shares of the decode shapes: each share's partial equals its four calls' bit
    for bit, and the two partials add up to the full layer."""
    _say("shares T=1")
    for first in (0, 5, 11):
        wl = synth.make(2, T=1, first_token=first)
        owner = moe.place_lpt(np.arange(wl.E, dtype=np.int64) % 7 + 1, 2)
        x = x_tensor(wl, torch)
        parts = []
        for share in (0, 1):
            g2l, l2g = moe.share_tables(owner, share)
            layer = make_layer(wl, l2g=l2g, g2l=g2l)
            got = _layer_call(layer, x, torch)
            ref = oracle_expect(wl, l2g=l2g, g2l=g2l)
            check_against_oracle(wl, got, ref, what=f"token {first} share {share}")
            _same_as_calls(got, _four_calls(layer, x, torch), _owned_rows(got, g2l), f"token {first} share {share}")
            parts.append(got["out"].astype(np.float64))
        full = _layer_call(make_layer(wl), x, torch)
        assert_close(parts[0] + parts[1], full["out"], f"token {first}: A + B vs the full layer")


def test_share_owning_none_of_the_token_experts(torch):
    """A share that owns none of the token's experts: no tile at all, the output is exactly zero,
    and the routing results are still stored."""
    _say("share with no owned slot")
    wl = synth.make(2, T=1)
    full = _layer_call(make_layer(wl), x_tensor(wl, torch), torch)
    chosen = set(full["ids"].reshape(-1).tolist())
    owner = np.array([1 if e in chosen else 0 for e in range(wl.E)], dtype=np.int32)
    g2l, l2g = moe.share_tables(owner, 0)
    got = _layer_call(make_layer(wl, l2g=l2g, g2l=g2l), x_tensor(wl, torch), torch)
    assert np.array_equal(got["ids"], full["ids"])
    assert got["w"].tobytes() == full["w"].tobytes()
    assert np.all(got["out"] == 0.0) and not np.any(np.signbit(got["out"]))


def test_consecutive_calls_on_one_buffer_set(torch):
    """Twelve decode steps through one set of buffers, with distinct tokens, then a repeat of the
    first: each equals a call on fresh buffers bit for bit."""
    _say("consecutive calls")
    from quantized_moe_routed_amd.layer import act_code
    wl = synth.make(2, T=12)
    layer = make_layer(wl)
    xs = [torch.from_numpy(np.ascontiguousarray(wl.x[t:t + 1])).cuda() for t in range(12)]
    b = layer.buffers(1, act_code(xs[0]))
    for t in list(range(12)) + [0]:
        got = _layer_call(layer, xs[t], torch, b)
        fresh = _layer_call(layer, xs[t], torch)
        assert got["out"].tobytes() == fresh["out"].tobytes(), f"step with token {t}"
        assert got["ids"].tobytes() == fresh["ids"].tobytes(), f"step with token {t}"
