"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Expert ids and groupings must match bit for bit; floating-point outputs
within max|d| <= 2e-3 max|ref| and rel-L2 <= 1e-4 (tests/helpers.py)."""
import sys

import numpy as np
import pytest

import oracle
import synth
import quantized_moe_routed_amd as moe
import helpers
from helpers import assert_close, oracle_expect, sha
from gpu_util import check_against_oracle, make_layer, run, torch_mod, x_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    return torch_mod()


def test_cfg1_tiny(torch):
    _say("cfg1 tiny T=4")
    wl = synth.make(1)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what="cfg1")


@pytest.mark.parametrize("T", [1, 5])
def test_cfg2_decode(torch, T):
    _say(f"cfg2 decode T={T}")
    wl = synth.make(2, T=T)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what=f"cfg2 T={T}")


def test_cfg3_batched_decode(torch):
    _say("cfg3 batched decode T=32")
    wl = synth.make(3)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what="cfg3")
    assert np.count_nonzero(got["counts"]) > 32      # the bias spreads load over many experts


def test_cfg3_ragged_tokens(torch):
    _say("cfg3 shapes, ragged T=37")
    wl = synth.make(3, T=37)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl, tokens=list(range(0, 37, 3))), what="cfg3 T=37")


def test_cfg5_shares_sum_to_full(torch):
    _say("cfg5 shares T=128")
    wl = synth.make(5)
    owner = moe.place_lpt(wl.load_hist, 2)
    assert np.array_equal(owner, oracle.place_lpt(wl.load_hist, 2))
    sample = list(range(0, 128, 4))
    full_ref = oracle_expect(wl, tokens=sample)
    parts = []
    for share in (0, 1):
        g2l, l2g = moe.share_tables(owner, share)
        assert len(l2g) == 128
        _say(f"cfg5 share {share}")
        got = run(make_layer(wl, l2g=l2g, g2l=g2l), wl, torch)
        ref = oracle_expect(wl, tokens=sample, l2g=l2g, g2l=g2l)
        check_against_oracle(wl, got, ref, what=f"cfg5 share {share}")
        # the permuted placement (local 0 != global 0) gives a bit-identical partial
        g2l_p, l2g_p = moe.share_tables(owner, share, wl.local_perm)
        assert np.any(l2g_p != l2g)
        got_p = run(make_layer(wl, l2g=l2g_p, g2l=g2l_p), wl, torch)
        assert got_p["out"].tobytes() == got["out"].tobytes()
        parts.append(got["out"])
    total = parts[0].astype(np.float64) + parts[1].astype(np.float64)
    assert_close(total[sample], full_ref["out"], "cfg5 partial A + partial B vs full")
    # and the sum against the GPU's own full layer, on every token
    full_gpu = run(make_layer(wl), wl, torch)
    assert_close(total, full_gpu["out"], "cfg5 A + B vs GPU full")


def test_repeat_runs_are_bit_identical(torch):
    _say("determinism cfg3 x5")
    wl = synth.make(3)
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    hashes = set()
    for _ in range(5):
        g = run(layer, wl, torch, x)
        hashes.add(sha(g["ids"], g["w"], g["counts"], g["offsets"], g["slot_list"], g["y"], g["out"]))
    assert len(hashes) == 1


def test_small_shapes_and_edge_cases(torch):
    _say("edge cases")
    # 5 router blocks (padded tree), fp32 router, Q8_0 experts, k = 1
    cfg = synth.custom(9, 160, 8, 96, 1, router_fmt=0)
    wl = synth.make(cfg)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what="H=160 k=1")
    assert np.all(got["w"] == 1.0)
    # Q2SM experts with Q8_0 router and bias, odd number of blocks in a row (H = 2080)
    cfg = synth.custom(6, 2080, 16, 224, 3, gate_fmt=2, up_fmt=2, down_fmt=2, router_fmt=1, bias="normal0.5")
    wl = synth.make(cfg)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what="H=2080 odd blocks")


def test_zero_router_ties_go_to_lower_ids(torch):
    _say("ties")
    wl = synth.make(1)
    wl.router = np.zeros_like(wl.router)          # fp32 zero router: every logit is 0
    got = run(make_layer(wl), wl, torch)
    assert np.array_equal(got["ids"], np.tile(np.arange(2), (wl.T, 1)))
    assert np.all(got["w"] == 0.5)


def test_t0_is_a_no_op(torch):
    _say("T=0")
    wl = synth.make(1, T=0)
    layer = make_layer(wl)
    x = torch.empty((0, wl.H), dtype=torch.float32, device="cuda")
    b = layer.buffers(0, 0)
    layer.run(x, b)
    torch.cuda.synchronize()
    assert b.counts.cpu().numpy().sum() == 0


def test_host_pointer_is_rejected(torch):
    _say("device check")
    wl = synth.make(1)
    layer = make_layer(wl)
    b = layer.buffers(wl.T, 0)
    host_x = np.ascontiguousarray(wl.x)
    with pytest.raises(moe.MoeError) as e:
        moe.route(host_x, 0, wl.T, wl.H, layer._router_q, None, wl.k, b.ids, b.w, b.route_ws,
                  b.route_ws.numel())
    assert e.value.status == moe.ERR_DEVICE


# ---- bf16 activations: the grouped MFMA GEMM ---------------------------------------------

def test_cfg4_prefill_shapes_small_batch(torch):
    _say("cfg4 prefill shapes, T=96 (tiles of 64 plus a ragged tail)")
    wl = synth.make(4, T=96)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl, tokens=list(range(0, 96, 5))), what="cfg4 T=96")


def _sample_tokens(ids, counts, n_each=6):
    """Tokens routed to the most loaded experts and to the least loaded (non-empty) ones."""
    order = np.argsort(-counts, kind="stable")
    heavy = [e for e in order if counts[e] > 0][:2]
    light = [e for e in order[::-1] if counts[e] > 0][:4]
    pick = []
    for e in heavy + light:
        toks = np.nonzero((ids == e).any(1))[0]
        pick += [int(t) for t in toks[:n_each]]
    pick += list(range(0, ids.shape[0], max(1, ids.shape[0] // 8)))
    return sorted(set(pick))


def test_cfg4_prefill_full_size(torch):
    _say("cfg4 prefill T=2048: ids/grouping for every token, sampled outputs, 5 runs bit-identical")
    wl = synth.make(4)
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    got = run(layer, wl, torch, x)
    ids, w, _ = oracle.route(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k)
    assert np.array_equal(got["ids"], ids), "expert ids differ"
    assert_close(got["w"], w, "weights")
    counts, offsets, slots = oracle.group(ids, wl.E)
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["slot_list"], slots)
    assert counts.max() > 2 * 64          # skewed load: the heaviest expert spans several tiles
    sample = _sample_tokens(ids, counts)
    _say(f"cfg4 oracle on {len(sample)} sampled tokens; max load {counts.max()}, distinct {np.count_nonzero(counts)}")
    ref = oracle_expect(wl, tokens=sample)
    check_against_oracle(wl, got, ref, what="cfg4 T=2048")
    h0 = sha(got["ids"], got["w"], got["counts"], got["offsets"], got["slot_list"], got["y"], got["out"])
    for rep in range(4):
        g = run(layer, wl, torch, x)
        assert sha(g["ids"], g["w"], g["counts"], g["offsets"], g["slot_list"], g["y"], g["out"]) == h0, rep


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_router_token_tiles_ragged(torch, act):
    """Batches of 64+ tokens take the token-tiled logits kernel (tiles of 4 tokens, a share of the
    tiles per workgroup row): T=133 leaves a partial tile and an uneven last share."""
    _say(f"router token tiles: T=133, H=4096, E=256, k=8, {act}")
    from quantized_moe_routed_amd.layer import act_code
    wl = synth.make(2 if act == "f32" else 4, T=133)
    layer = make_layer(wl)
    x = x_tensor(wl, torch)
    b = layer.buffers(wl.T, act_code(x))
    layer.route(x, b)
    torch.cuda.synchronize()
    ids, w, _ = oracle.route(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k)
    assert np.array_equal(b.ids.cpu().numpy(), ids), "expert ids differ"
    assert_close(b.w.cpu().numpy(), w, "weights")


def test_bf16_small_shapes_and_share(torch):
    _say("bf16 small shapes: H=128, I=192, E=8, k=3, T=23; then an owned share and its complement")
    cfg = synth.custom(23, 128, 8, 192, 3, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1, act="bf16",
                       bias="normal0.5", name="bf16_small")
    wl = synth.make(cfg)
    got = run(make_layer(wl), wl, torch)
    check_against_oracle(wl, got, oracle_expect(wl), what="bf16 small")
    owner = np.array([0, 1, 1, 0, 1, 0, 0, 1], np.int32)
    parts = []
    for share in (0, 1):
        g2l, l2g = moe.share_tables(owner, share, np.array([3, 1, 7, 0, 5, 2, 6, 4], np.int32))
        assert l2g[0] != 0 or share == 1
        gs = run(make_layer(wl, l2g=l2g, g2l=g2l), wl, torch)
        check_against_oracle(wl, gs, oracle_expect(wl, l2g=l2g, g2l=g2l), what=f"bf16 share {share}")
        parts.append(gs["out"].astype(np.float64))
    assert_close(parts[0] + parts[1], got["out"], "bf16 share A + share B vs full")


# ---- large tiles: experts with at least moe_large_tile_min(T) slots -------------------------

_LARGE_CASES = {
    # fp32 activations (hi + lo planes), 2-bit everywhere, a partly filled last code unit (H = 320)
    "f32_q2sm": (64, 320, 8, 192, 2, dict(gate_fmt=2, up_fmt=2, down_fmt=2, router_fmt=1, act="f32")),
    # fp32 activations, Q8_0 everywhere, fp32 router
    "f32_q8": (64, 256, 6, 320, 2, dict(gate_fmt=1, up_fmt=1, down_fmt=1, router_fmt=0, act="f32")),
    # bf16 activations, Q8_0 gate/up, 2-bit down
    "bf16_q8_q2sm": (48, 192, 8, 256, 3, dict(gate_fmt=1, up_fmt=1, down_fmt=2, router_fmt=1, act="bf16")),
    # several full tiles of 128 slots per expert plus ragged tails, next to one small expert
    "f32_multi_tile": (300, 128, 4, 128, 2, dict(gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1, act="f32")),
    # an odd number of blocks per row (H = 2080: 65 blocks), I = 96 (a partial column tile and a
    # partly filled 2-bit unit in the down projection)
    "f32_odd_blocks": (40, 2080, 6, 96, 2, dict(gate_fmt=1, up_fmt=1, down_fmt=2, router_fmt=1, act="f32")),
    # a batch of 33 tokens (the smallest batches with large tiles): an expert of all 33 tokens on a
    # large tile beside one of 32 slots on 4 small tiles
    "f32_t33": (33, 256, 4, 128, 3, dict(gate_fmt=2, up_fmt=2, down_fmt=2, router_fmt=1, act="f32")),
    # 256 tokens without router bias (the smallest batches with large tiles from 12 slots):
    # experts of 12-14 slots on large tiles, of 9-11 on two small tiles, the rest on one
    "f32_t256_even": (256, 256, 64, 128, 2, dict(gate_fmt=2, up_fmt=2, down_fmt=2, router_fmt=1, act="f32",
                                                 bias=None)),
}


@pytest.mark.parametrize("name", sorted(_LARGE_CASES))
def test_large_tiles_against_oracle(torch, name):
    T, H, E, I, k, kw = _LARGE_CASES[name]
    _say(f"large tiles {name}: T={T} H={H} E={E} I={I} k={k}")
    kw = dict(kw)
    wl = synth.make(synth.custom(T, H, E, I, k, bias=kw.pop("bias", "zipf1.1"), name=name, **kw))
    got = run(make_layer(wl), wl, torch)
    counts = got["counts"]
    lmin = moe.large_tile_min(T)
    assert lmin > 0 and counts.max() >= lmin and ((counts > 0) & (counts < lmin)).any()   # both tile kinds
    if name == "f32_multi_tile":
        assert counts.max() > 2 * 128
    check_against_oracle(wl, got, oracle_expect(wl), what=f"large {name}")


# slots per expert around the large kernel's row-group and tile edges (a batch of 429 tokens, one
# slot each, so experts of 12 or more slots take large tiles): 32 and 33 (one and two 32-row
# fragments, contraction split between the row groups), 64 (the split's largest tile), 65 and 96
# (second row group on one fragment), 129 (a full tile and a split tile of one row), 10 (two small
# tiles), 0
_EDGE_COUNTS = [32, 33, 64, 65, 96, 129, 10, 0]


@pytest.mark.parametrize("act,fm", [("f32", (2, 2, 1)), ("bf16", (1, 1, 2))])
def test_large_tile_row_edges(torch, act, fm):
    """Expert loads set by hand at the large kernel's row-group edges: every y_slot row equals the
    oracle's expert output for its slot, within tolerance."""
    T, E = sum(_EDGE_COUNTS), len(_EDGE_COUNTS)
    _say(f"large-tile row edges {act} fmts={fm}: T={T} counts={_EDGE_COUNTS}")
    assert moe.large_tile_min(T) == 12
    wl = synth.make(synth.custom(T, 256, E, 128, 1, gate_fmt=fm[0], up_fmt=fm[1], down_fmt=fm[2], router_fmt=1,
                                 act=act, name=f"edges_{act}"))
    ids = np.repeat(np.arange(E, dtype=np.int32), _EDGE_COUNTS)
    ids = ids[np.random.default_rng(7).permutation(T)].reshape(T, 1)
    layer = make_layer(wl)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    b = layer.buffers(T, act_code(x))
    b.ids.copy_(torch.from_numpy(ids))
    layer.group(b)
    layer.forward(x, b)
    torch.cuda.synchronize()
    assert np.array_equal(b.counts.cpu().numpy(), np.array(_EDGE_COUNTS))
    rows = oracle.forward_slots(helpers.fmts(wl), wl.gate, wl.up, wl.down, wl.x, ids, range(T))
    ref = np.stack([rows[s] for s in range(T)])
    assert_close(b.y_slot.cpu().numpy()[:T], ref, f"edges {act} y_slot")


def _run_both(layer, wl, torch):
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    outs = []
    for fused in (False, True):
        b = layer.buffers(wl.T, act_code(x))
        (layer.run if fused else layer.run_calls)(x, b)
        torch.cuda.synchronize()
        outs.append([b.ids.cpu().numpy(), b.w.cpu().numpy(), b.counts.cpu().numpy(), b.offsets.cpu().numpy(),
                     b.slot_list.cpu().numpy()[: wl.T * wl.k], b.y_slot.cpu().numpy(), b.out.cpu().numpy()])
    return outs


@pytest.mark.parametrize("cfg,T", [(2, 1), (2, 8), (3, 9), (3, 32), (4, 20)])
def test_layer_call_equals_the_four_calls(torch, cfg, T):
    """moe_layer_forward (one launch for selection, grouping, tiles and operands up to 8 tokens)
    gives the four calls' results bit for bit, on both sides of the 8-token switch."""
    _say(f"layer call vs four calls: cfg{cfg} T={T}")
    wl = synth.make(cfg, T=T)
    calls, fused = _run_both(make_layer(wl), wl, torch)
    for name, a, b in zip(("ids", "w", "counts", "offsets", "slot_list", "y_slot", "out"), calls, fused):
        assert np.array_equal(a, b), f"{name} differs between the layer call and the four calls"


@pytest.mark.parametrize("H", [8192, 16384])
def test_router_wide_rows(torch, H):
    """Wide router rows give the small-batch logits kernel 8 and 16 aligned ranges of 32 blocks
    (the top-k launch adds up to 32 ranges, the selection inside the gate/up launch up to 8): the
    router call's ids equal the oracle's and its weights are within tolerance; at H=8192 the
    one-token layer call, which selects inside the gate/up launch, matches the oracle too."""
    from quantized_moe_routed_amd.layer import DeviceMatrix
    _say(f"router with wide rows: H={H}")
    T, E, k = 3, 64, 4
    wl = synth.make(synth.custom(T, H, E, 128, k, name=f"wide{H}"), experts=False)
    ref_ids, ref_w, _ = oracle.route(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k)
    R = DeviceMatrix(wl.cfg.router_fmt, wl.router[0], 1, E, H, "cuda")
    rws, _, _ = moe.workspace_size(T, H, 128, k, E, E, moe.ACT_F32)
    ws = torch.empty(max(rws, 16), dtype=torch.uint8, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    moe.route(torch.from_numpy(wl.x).cuda(), moe.ACT_F32, T, H, R.qmat(), None, k, ids, w, ws, ws.numel())
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref_ids), f"ids, H={H}"
    assert_close(w.cpu().numpy(), ref_w, what=f"router weights H={H}")
    if H <= 8192:
        wl1 = synth.make(synth.custom(1, H, 16, 256, k, bias="zipf1.1", name=f"wide{H}_t1"))
        check_against_oracle(wl1, run(make_layer(wl1), wl1, torch), oracle_expect(wl1), what=f"one token H={H}")


@pytest.mark.parametrize("E,k", [(8, 8), (40, 2), (100, 8), (256, 1), (256, 8), (256, 9), (300, 8), (1024, 8)])
def test_topk_ties_against_a_stable_sort(torch, E, k):
    """Top-k where most choices cross a tie: router bytes of zero (scale 0) make every logit equal
    to its bias, drawn from four values.  The layer call (selection inside the gate/up launch up to
    256 experts, in the front launch above) and the four calls must both give the k largest with
    ties to the lower index, i.e. a stable sort of (-bias, index), and the normalised sigmoids."""
    T = 3
    _say(f"top-k ties: E={E}, k={k}")
    wl = synth.make(synth.custom(T, 256, E, 64, k, name=f"ties_E{E}_k{k}"))
    wl.router[:] = 0
    rng = np.random.default_rng(1000 * E + k)
    wl.bias = rng.choice(np.array([-0.5, 0.0, 0.25, 1.0], np.float32), size=E)
    order = np.lexsort((np.arange(E), -wl.bias.astype(np.float64)))[:k]
    sg = 1.0 / (1.0 + np.exp(-wl.bias[order].astype(np.float64)))
    calls, fused = _run_both(make_layer(wl), wl, torch)
    for got in (calls, fused):
        assert np.array_equal(got[0].reshape(T, k), np.tile(order, (T, 1))), f"ids, E={E}, k={k}"
        assert_close(got[1].reshape(T, k), np.tile(sg / sg.sum(), (T, 1)), what=f"weights E={E} k={k}")


@pytest.mark.parametrize("cfg,T", [(3, 32), (5, 128)])
def test_down_tiles_of_eight_beside_gateup_tiles_of_four(torch, cfg, T):
    """fp32 activations at H = 4096: the gate/up projection takes small tiles of 4 slots (its staging
    of 8 rows would not let two workgroups share a compute unit) while the down projection, whose
    staging of 8 rows fits (K = I = 2048), takes tiles of its own of 8.  The y_slot rows of every
    expert of 5 to 8 slots (two gate/up tiles, one down tile) equal the oracle's expert outputs."""
    _say(f"down tiles of 8 beside gate/up tiles of 4: cfg{cfg} T={T}")
    wl = synth.make(cfg, T=T)
    g2l = l2g = None
    if cfg == 5:
        owner = moe.place_lpt(wl.load_hist, 2)
        g2l, l2g = moe.share_tables(owner, 0)
    layer = make_layer(wl, l2g=l2g, g2l=g2l)
    got = run(layer, wl, torch)
    counts, offsets, slots = got["counts"], got["offsets"], got["slot_list"]
    owned = np.ones(wl.E, bool) if g2l is None else np.asarray(g2l) >= 0
    mid = [e for e in range(wl.E) if owned[e] and 5 <= counts[e] <= 8]
    assert mid, "no owned expert of 5 to 8 slots"
    pick = [int(sl) for e in mid[:6] for sl in slots[offsets[e]:offsets[e + 1]]]
    gate, up, down = (wl.gate, wl.up, wl.down) if l2g is None else (wl.gate[l2g], wl.up[l2g], wl.down[l2g])
    rows = oracle.forward_slots(helpers.fmts(wl), gate, up, down, wl.x, got["ids"], pick,
                                g2l=None if g2l is None else np.asarray(g2l))
    ref = np.stack([rows[sl] for sl in pick])
    assert_close(got["y"][pick], ref, f"cfg{cfg} y rows of experts of 5-8 slots")


@pytest.mark.parametrize("T,k,E", [(300, 8, 256), (2049, 8, 64), (129, 8, 1024), (4096, 1, 3)])
def test_group_over_several_chunks(torch, T, k, E):
    """The grouping launch takes 1024 slots per workgroup: batches of several chunks with a ragged
    last one, ids outside [0, E) (left out) and experts that receive nothing.  counts, offsets and
    the slot list equal a stable sort of the valid slots by expert (numpy's stable argsort), and
    slot_list entries past the valid slots are left untouched."""
    _say(f"grouping over chunks: T={T} k={k} E={E}")
    rng = np.random.default_rng(T * 31 + k)
    n = T * k
    ids = rng.integers(0, E, size=n).astype(np.int32)
    ids[rng.random(n) < 0.02] = -1                 # left out
    ids[rng.random(n) < 0.02] = E + 5              # left out
    if E >= 64:
        ids[(ids % 7) == 3] = 0                    # a heavy expert; others receive nothing
    valid = (ids >= 0) & (ids < E)
    counts_ref = np.bincount(ids[valid], minlength=E).astype(np.int32)
    offsets_ref = np.concatenate([[0], np.cumsum(counts_ref)]).astype(np.int32)
    vs = np.nonzero(valid)[0]
    order_ref = vs[np.argsort(ids[vs], kind="stable")].astype(np.int32)
    d = torch.device("cuda")
    ids_d = torch.from_numpy(ids).to(d)
    counts = torch.full((E,), -9, dtype=torch.int32, device=d)
    offsets = torch.full((E + 1,), -9, dtype=torch.int32, device=d)
    slots = torch.full((n,), -9, dtype=torch.int32, device=d)
    moe.group_tokens(ids_d, T, k, E, counts, offsets, slots)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), counts_ref)
    assert np.array_equal(offsets.cpu().numpy(), offsets_ref)
    got = slots.cpu().numpy()
    assert np.array_equal(got[: len(vs)], order_ref)
    assert np.all(got[len(vs):] == -9)


@pytest.mark.parametrize("k", [1, 5, 8, 9, 17])
def test_combine_alone(torch, k):
    """moe_combine by itself, with and without an owner table (some experts unowned, one id past the
    expert range), H=1000 leaving a partial workgroup.  Dyadic inputs (y in steps of 2^-10 below 1,
    w in steps of 2^-8) make every product and partial sum exact in fp32, so the sum over the owned
    slots is known exactly; random inputs are checked against a float64 sum."""
    _say(f"combine alone: k={k}")
    rng = np.random.default_rng(100 + k)
    T, H, E = 3, 1000, 40
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, k - 1] = E + 3
    g2l = np.where(rng.random(E) < 0.6, np.arange(E), -1).astype(np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for exact in (True, False):
        if exact:
            y = (rng.integers(-1000, 1001, size=(T * k, H)) / 1024.0).astype(np.float32)
            w = (rng.integers(1, 256, size=(T, k)) / 256.0).astype(np.float32)
        else:
            y = rng.standard_normal((T * k, H)).astype(np.float32)
            w = rng.random((T, k)).astype(np.float32)
        for table in (None, g2l):
            own = np.ones((T, k), bool) if table is None else (ids < E) & (table[np.minimum(ids, E - 1)] >= 0)
            ref = np.einsum("tj,tjh->th", (w * own).astype(np.float64), y.reshape(T, k, H).astype(np.float64))
            out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
            moe.combine(dev(y), dev(w), dev(ids), None if table is None else dev(table), T, k, H, E, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            if exact:
                assert np.array_equal(got, ref.astype(np.float32)), f"k={k}, table={table is not None}"
            else:
                assert_close(got, ref, what=f"combine k={k}")


@pytest.mark.parametrize("I,k", [(2304, 8), (4096, 8), (1280, 8), (2048, 3)])
def test_layer_call_one_token_down_widths(torch, I, k):
    """One token with 2-bit down weights at several expert widths: the down launch's waves take one
    code unit each up to I=2048 (I=1280: five units, three waves empty; k=3: three tiles) and one
    or two beyond (I=2304, nine units: waves with one unit and waves with none)."""
    _say(f"layer call vs four calls: one token, I={I}, k={k}")
    wl = synth.make(synth.custom(1, 2048, 64, I, k, gate_fmt=synth.FMT_Q2SM, up_fmt=synth.FMT_Q2SM,
                                 down_fmt=synth.FMT_Q2SM, bias="zipf1.1", name=f"down_w{I}_k{k}"))
    layer = make_layer(wl)
    calls, fused = _run_both(layer, wl, torch)
    for name, a, b in zip(("ids", "w", "counts", "offsets", "slot_list", "y_slot", "out"), calls, fused):
        assert np.array_equal(a, b), f"{name} differs between the layer call and the four calls"
    check_against_oracle(wl, run(layer, wl, torch), oracle_expect(wl), what=f"one token I={I} k={k}")


@pytest.mark.parametrize("T", [1, 5, 24])
def test_layer_call_owned_share(torch, T):
    """The layer call with an owned-expert table (a share of the experts): the four calls' partial,
    for one token, a batch that the expert launch routes by itself, and one routed by separate
    launches."""
    _say(f"layer call vs four calls: cfg5 share, T={T}")
    wl = synth.make(5, T=T)
    owner = moe.place_lpt(np.arange(wl.E, dtype=np.int64) % 7 + 1, 2)
    g2l, l2g = moe.share_tables(owner, 0)
    calls, fused = _run_both(make_layer(wl, l2g=l2g, g2l=g2l), wl, torch)
    for name, a, b in zip(("ids", "w", "counts", "offsets", "slot_list", "y_slot", "out"), calls, fused):
        assert np.array_equal(a, b), f"{name} differs between the layer call and the four calls"


@pytest.mark.parametrize("name", ["ffn_gateup", "combine"])
def test_kernel_trace_records_each_launch(torch, name):
    """moe_trace_kernel_every records launches 0, 2, 4 of a kernel: stamped by the launch itself
    (expert kernels) or by events on the stream around it (the others); each recorded interval is
    positive and no longer than the whole layer call that contains it."""
    _say(f"kernel trace {name}")
    wl = synth.make(3, T=32)
    layer = make_layer(wl)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    b = layer.buffers(wl.T, act_code(x))
    layer.run(x, b)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with moe.KernelTrace(name, 4, 2) as tr:
        t0.record()
        for _ in range(5):
            layer.run(x, b)
        t1.record()
    times = tr.times_ms()
    assert tr.count.value == 3 and len(times) == 3
    total = t0.elapsed_time(t1)
    assert all(0.0 < t < total for t in times), (times, total)



def test_route_table_top_k_rows_match_route(torch):
    """A device table whose row t is token t's top k from moe_route: moe_route_table returns the
    same ids and, bit for bit, the same weights."""
    _say("route_table vs route: cfg3 T=32")
    wl = synth.make(3, T=32)
    layer = make_layer(wl)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    b = layer.buffers(wl.T, act_code(x))
    layer.route(x, b)
    torch.cuda.synchronize()
    ids, w = b.ids.clone(), b.w.clone()
    b.ids.zero_()
    b.w.zero_()
    layer.route_table(x, b, torch.arange(wl.T, dtype=torch.int32, device="cuda"), ids)
    torch.cuda.synchronize()
    assert torch.equal(b.ids, ids)
    assert torch.equal(b.w.view(torch.int32), w.view(torch.int32))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_route_table_layer_against_oracle(torch, act):
    """The layer with table routing (route_table, group, experts, combine) against the oracle's
    table route, per-slot experts and combine: ids and grouping exact, weights and output within
    tolerance."""
    T, H, E, I, k, V = 40, 256, 32, 128, 4, 64
    _say(f"route_table layer {act}: T={T} E={E} k={k} V={V}")
    wl = synth.make(synth.custom(T, H, E, I, k, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1, act=act,
                                 bias="zipf1.1", name=f"table_{act}"))
    table = synth.route_table(0, V, E, k)
    tok = synth.token_ids(0, T, V)
    moe.table_check(table, E)
    layer = make_layer(wl)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    b = layer.buffers(T, act_code(x))
    layer.run_table(x, b, torch.from_numpy(tok).cuda(), torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    ids, w = oracle.route_table(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, tok, table)
    assert np.array_equal(b.ids.cpu().numpy(), ids)
    assert_close(b.w.cpu().numpy(), w, "table weights")
    counts, offsets, slots = oracle.group(ids, E)
    assert np.array_equal(b.counts.cpu().numpy(), counts)
    assert np.array_equal(b.slot_list.cpu().numpy()[: T * k], slots)
    rows = oracle.forward_slots(helpers.fmts(wl), wl.gate, wl.up, wl.down, wl.x, ids, range(T * k))
    y = np.stack([rows[s] for s in range(T * k)])
    assert_close(b.y_slot.cpu().numpy()[: T * k], y, "table y_slot")
    assert_close(b.out.cpu().numpy(), oracle.combine(y, w, ids, None), "table out")



@pytest.mark.parametrize("T,act,sfmt", [(1, "f32", 1), (8, "f32", 1), (32, "f32", 1), (40, "f32", 1), (300, "f32", 1),
                                         (40, "bf16", 1), (8, "f32", 2), (300, "f32", 2)])
def test_shared_expert_adds_to_the_routed_output(torch, T, act, sfmt):
    """The layer's routed output plus the shared expert (every token through one Q8_0 or 2-bit
    expert) against the oracle's routed output plus its per-token shared expert.  The one expert
    takes all T slots: 1 token runs on one-slot tiles, 8 and 32 on tiles of several slots, 40 and
    300 (moe_large_tile_min: 33 and 12) on large tiles."""
    H, E, I, k, Is = 256, 8, 128, 2, 160
    _say(f"shared expert {act} fmt {sfmt}: T={T} H={H} I_shared={Is}")
    wl = synth.make(synth.custom(T, H, E, I, k, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1, act=act,
                                 name=f"shared_{act}"))
    sg, su, sd = synth.shared_expert(0, H, Is, sfmt)
    from quantized_moe_routed_amd.layer import SharedExpert
    shared = SharedExpert(H, Is, sfmt, sg, su, sd)
    layer = make_layer(wl)
    from quantized_moe_routed_amd.layer import act_code
    x = x_tensor(wl, torch)
    b = layer.buffers(T, act_code(x))
    layer.run(x, b)
    shared.add_to(x, b.out)
    torch.cuda.synchronize()
    ref = oracle_expect(wl)["out"].astype(np.float64) + oracle.shared_expert((sfmt,) * 3, sg, su, sd, wl.x)
    assert_close(b.out.cpu().numpy(), ref, f"shared {act} T={T} out")


@pytest.mark.parametrize("T,H", [(24, 3104), (20, 2304)])
def test_unit_by_unit_gateup_odd_widths(torch, T, H):
    """2-bit gate/up of several slots with fp32 activations where the whole staging of 8 rows would
    not let two workgroups share a compute unit, so each wave stages its rows a code unit at a
    time: H = 3104 (97 blocks: 13 units, the last of one block; waves of two, one or no units) and
    H = 2304 (9 whole units: waves of two units, of one, and without), with tiles of up to 8 slots
    (zipf routing gives some experts more than 8)."""
    _say(f"unit-by-unit gate/up: T={T} H={H}")
    assert moe.large_tile_min(T) == 0
    wl = synth.make(synth.custom(T, H, 16, 128, 4, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1, act="f32",
                                 bias="zipf1.1", name=f"unitwise_{H}"))
    got = run(make_layer(wl), wl, torch)
    assert got["counts"].max() > 8
    check_against_oracle(wl, got, oracle_expect(wl), what=f"unit-by-unit H={H}")
