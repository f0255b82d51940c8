"""Pins of the CPU oracle against facts it does not compute itself.

Each test fixes the oracle to something independent of its own code: a
closed form, a hand-worked rounding case, a library routine (numpy fp64
matrix products in ``oracle/brute.py``), brute force on tiny inputs, the
invariants of expert ownership, or the numbers a page prints.
"""
import math
import os
import struct

import numpy as np
import pytest

import oracle
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(v: float) -> bytes:
    return struct.pack("<e", v)


def q8_block(d: float, q) -> bytes:
    return f16(d) + struct.pack("<32b", *q)


def q2_block(d: float, m: float, codes) -> bytes:
    qs = bytearray(8)
    for i, c in enumerate(codes):
        qs[i // 4] |= (c & 3) << (2 * (i % 4))
    return f16(d) + f16(m) + bytes(qs)


def f32_row(vals) -> np.ndarray:
    return np.frombuffer(np.asarray(vals, dtype=np.float32).tobytes(), dtype=np.uint8)


# ----------------------------------------------------------------- dequant
def test_q2sm_block_closed_form():
    # d = 1, m = -2, codes 0,1,2,3 repeating: values -2, -1, 0, 1
    row = np.frombuffer(q2_block(1.0, -2.0, [i % 4 for i in range(32)]), dtype=np.uint8)
    want = np.array([(i % 4) - 2.0 for i in range(32)])
    assert np.array_equal(oracle.dequant_rows(2, row, 32)[0], want)
    assert np.array_equal(brute.decode(2, row[None], 32)[0], want)


def test_q2sm_bit_order():
    # only value 5 has code 3 -> byte 1, bits 2..3
    codes = [0] * 32
    codes[5] = 3
    blk = q2_block(0.5, 0.25, codes)
    assert blk[4 + 1] == 0b00001100
    v = oracle.dequant_rows(2, np.frombuffer(blk, np.uint8), 32)[0]
    assert v[5] == 1.75 and np.all(np.delete(v, 5) == 0.25)


def test_q8_0_block_closed_form():
    q = [64, -127, 0, 1] + [0] * 28
    row = np.frombuffer(q8_block(2.0 ** -7, q), dtype=np.uint8)
    v = oracle.dequant_rows(1, row, 32)[0]
    assert v[0] == 0.5 and v[1] == -127 / 128 and v[2] == 0.0 and v[3] == 2.0 ** -7
    assert np.array_equal(v, brute.decode(1, row[None], 32)[0])


def test_subnormal_fp16_scale():
    row = np.frombuffer(struct.pack("<H", 1) + struct.pack("<32b", *([3] * 32)), np.uint8)
    assert np.all(oracle.dequant_rows(1, row, 32)[0] == 3 * 2.0 ** -24)


@pytest.mark.parametrize("fmt", [1, 2])
def test_encode_decode_round_trip_bound(fmt):
    rows, cols = 64, 256
    stream = 99 << 20
    enc = synth.quant_matrices(7, stream, 1, rows, cols, fmt)[0]
    v = synth.normal(7, stream, rows * cols, synth.W_SIGMA).reshape(rows, cols).astype(np.float64)
    deq = oracle.dequant_rows(fmt, enc, cols)
    vb = v.reshape(rows, cols // 32, 32)
    err = np.abs(deq - v).reshape(rows, cols // 32, 32)
    if fmt == 1:
        d = np.abs(vb).max(-1) / 127.0
        bound = d * (0.5 + 127 * 2.0 ** -11) + 1e-12
    else:
        lo, hi = vb.min(-1), vb.max(-1)
        d = (hi - lo) / 3.0
        bound = 0.5 * d * (1 + 2.0 ** -10) + np.abs(lo) * 2.0 ** -11 + 3 * d * 2.0 ** -11 + 1e-12
    assert np.all(err <= bound[..., None])


# ----------------------------------------------------------------- router
def _f32_router_row(vals):
    return f32_row(vals)


def test_router_tree_order_pairs_adjacent_blocks():
    # block partials r = [1e8, 1, -1e8, 1]: the adjacent-pair tree gives
    # (1e8 + 1) + (-1e8 + 1) = 1e8 - 1e8 = 0 in fp32 (1e8 + 1 rounds to 1e8);
    # a left-to-right sum would give 1, pairing (r0 + r2) + (r1 + r3) gives 2.
    H = 128
    x = np.zeros(H, np.float32)
    w = np.zeros(H, np.float32)
    for b, val in enumerate([1e8, 1.0, -1e8, 1.0]):
        x[32 * b] = val
        w[32 * b] = 1.0
    assert oracle.router_logit(0, _f32_router_row(w), x) == 0.0


def test_router_tree_carries_odd_tail():
    # r = [1, 1e8, -1e8]: ((1 + 1e8) + carried -1e8) = 0, right-nested would give 1
    x = np.zeros(96, np.float32)
    w = np.zeros(96, np.float32)
    for b, val in enumerate([1.0, 1e8, -1e8]):
        x[32 * b], w[32 * b] = val, 1.0
    assert oracle.router_logit(0, _f32_router_row(w), x) == 0.0
    # r = [1e8, 1, -1e8, 1, 1]: ((1e8+1) + (-1e8+1)) + 1 = 1; left-to-right gives 2
    x = np.zeros(160, np.float32)
    w = np.zeros(160, np.float32)
    for b, val in enumerate([1e8, 1.0, -1e8, 1.0, 1.0]):
        x[32 * b], w[32 * b] = val, 1.0
    assert oracle.router_logit(0, _f32_router_row(w), x) == 1.0


def test_router_block_chain_is_fused():
    # -(1 + 2^-11) * 1 + (1 + 2^-12)^2 = 2^-24 exactly with fused multiply-add;
    # rounding the product first gives 0
    x = np.zeros(32, np.float32)
    w = np.zeros(32, np.float32)
    w[0], x[0] = -(1 + 2.0 ** -11), 1.0
    w[1] = x[1] = 1 + 2.0 ** -12
    assert oracle.router_logit(0, _f32_router_row(w), x) == 2.0 ** -24


def test_router_q8_scale_multiplies_block_sum():
    # integer x, q: the block sum is exact; z = d * p with d = 2^-7 exact
    rng = np.random.default_rng(1)
    q = rng.integers(-127, 128, 64)
    x = rng.integers(-8, 9, 64).astype(np.float32)
    row = np.frombuffer(q8_block(2.0 ** -7, q[:32]) + q8_block(2.0 ** -7, q[32:]), np.uint8)
    z = oracle.router_logit(1, row, x)
    assert z == float(np.dot(q, x)) / 128.0
    assert oracle.router_logit(1, row, x, bias_e=0.25) == np.float32(z) + np.float32(0.25)


def test_router_matches_fp64_brute_force():
    wl = synth.make(synth.custom(16, 512, 16, 64, 4, router_fmt=1, bias="normal0.5"))
    ids, w, z = oracle.route(wl.x, 1, wl.router[0], wl.bias, 4)
    ref = brute.layer(wl.x, 1, wl.router[0], wl.bias, 4, (1, 1, 1), wl.gate, wl.up, wl.down)
    scale = np.abs(wl.x.astype(np.float64)) @ np.abs(brute.decode(1, wl.router[0], 512)).T
    assert np.all(np.abs(z - ref["z"]) <= 1e-5 * scale + 1e-6)
    clear = ref["margin"] > 1e-4
    assert clear.sum() >= 12
    assert np.array_equal(ids[clear], ref["ids"][clear])


# ----------------------------------------------------------------- select / weights
def test_zero_router_selects_lowest_ids_with_equal_weights():
    E, H = 8, 64
    router = np.frombuffer(b"".join(q8_block(0.0, [0] * 32) for _ in range(E * H // 32)), np.uint8)
    x = synth.normal(3, 1, 5 * H).reshape(5, H)
    for k, wk in [(1, 1.0), (2, 0.5), (3, np.float32(1 / 3)), (8, 0.125)]:
        ids, w, _ = oracle.route(x, 1, router.reshape(E, -1), None, k)
        assert np.array_equal(ids, np.tile(np.arange(k), (5, 1)))
        assert np.all(w == wk)


def test_selection_is_permutation_equivariant():
    wl = synth.make(synth.custom(8, 256, 16, 64, 3, router_fmt=1, bias="normal0.5"))
    r = wl.router[0]
    ids, _, z = oracle.route(wl.x, 1, r, wl.bias, 3)
    perm = np.random.default_rng(5).permutation(16)          # new expert i = old perm[i]
    ids_p, _, z_p = oracle.route(wl.x, 1, r[perm], wl.bias[perm], 3)
    inv = np.argsort(perm)
    assert np.array_equal(z_p, z[:, perm])
    assert np.array_equal(ids_p, inv[ids])                   # no ties in these draws


def test_weights_sum_to_one_and_order():
    wl = synth.make(2, T=3, experts=False)
    ids, w, z = oracle.route(wl.x, 1, wl.router[0], None, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 8 * 2.0 ** -24)
    zs = np.take_along_axis(z, ids, 1)
    assert np.all(np.diff(zs, axis=1) <= 0)
    assert np.all(np.diff(w, axis=1) <= 0)                   # sigmoid is increasing
    ids1, w1, _ = oracle.route(wl.x, 1, wl.router[0], None, 1)
    assert np.all(w1 == 1.0) and np.array_equal(ids1[:, 0], ids[:, 0])


# ----------------------------------------------------------------- group
def test_group_matches_sorted():
    rng = np.random.default_rng(2)
    for T, k, E in [(1, 8, 256), (37, 3, 16), (0, 2, 8), (200, 8, 256)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        counts, offsets, slots = oracle.group(ids, E)
        ref = [s for _, s in sorted((int(ids.flat[s]), s) for s in range(T * k))]
        assert slots.tolist() == ref
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)


def test_imbalance_closed_form_reproduces_page_numbers():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "imbalance_arc_pr89.txt")) if l[0] != "#"]
    E, k = 256, 6
    for B, pct, dec in rows:
        distinct = E * (1 - (1 - k / E) ** int(B))
        assert round(100 * (E / distinct - 1), int(dec)) == float(pct)


def test_group_counts_distinct_experts_like_closed_form():
    # uniformly random top-k sets: mean number of non-empty groups -> E(1-(1-k/E)^B)
    rng = np.random.default_rng(3)
    E, k, B, trials = 256, 6, 64, 300
    D = []
    for _ in range(trials):
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(B)]).astype(np.int32)
        counts, _, _ = oracle.group(ids, E)
        D.append((counts > 0).sum())
    D = np.array(D, dtype=np.float64)
    want = E * (1 - (1 - k / E) ** B)
    assert abs(D.mean() - want) <= 4 * D.std() / math.sqrt(trials)


# ----------------------------------------------------------------- FFN
def test_expert_matches_numpy_products():
    wl = synth.make(synth.custom(3, 256, 4, 128, 1, gate_fmt=2, up_fmt=2, down_fmt=1))
    fm = (2, 2, 1)
    Y = brute.all_experts(fm, wl.gate, wl.up, wl.down, wl.x)
    for e in range(4):
        for t in range(3):
            y = oracle.expert(fm, wl.gate[e], wl.up[e], wl.down[e], wl.x[t])
            assert np.allclose(y, Y[e, t], rtol=1e-12, atol=1e-14 * np.abs(Y).max())


def test_expert_closed_form_constant_rows():
    H, I = 64, 96
    qa, qb, qc = 5, -3, 7                  # values a = q/128 with d = 2^-7
    def mat(rows, cols, q):
        return np.frombuffer(b"".join(q8_block(2.0 ** -7, [q] * 32) for _ in range(rows * cols // 32)),
                             np.uint8).reshape(rows, -1)
    x = synth.normal(4, 2, H)
    S = float(np.sum(x.astype(np.float64)))
    a, b, c = qa / 128, qb / 128, qc / 128
    g, u = a * S, b * S
    want = c * I * (g / (1 + math.exp(-g))) * u
    y = oracle.expert((1, 1, 1), mat(I, H, qa), mat(I, H, qb), mat(H, I, qc), x)
    assert np.allclose(y, want, rtol=1e-12)


def test_shared_expert_closed_form_per_token():
    """oracle.shared_expert on a one-expert stack with constant rows (Q8_0 gate/up/down, and 2-bit
    ones, value d q + m with every code equal): row t is c I SiLU(a S_t) (b S_t) in every column,
    S_t the sum of token t's activations, for tokens of very different sizes."""
    H, I, T = 64, 96, 5

    def q8(rows, cols, q):
        return np.frombuffer(b"".join(q8_block(2.0 ** -7, [q] * 32) for _ in range(rows * cols // 32)),
                             np.uint8).reshape(1, rows, -1)

    def q2(rows, cols, d, m, q):
        return np.frombuffer(b"".join(q2_block(d, m, [q] * 32) for _ in range(rows * cols // 32)),
                             np.uint8).reshape(1, rows, -1)

    x = (synth.normal(4, 3, T * H).reshape(T, H) * np.array([1e-3, 0.1, 1.0, 10.0, 300.0])[:, None]).astype(np.float32)
    S = x.astype(np.float64).sum(1)
    cases = [((1, 1, 1), q8(I, H, 5), q8(I, H, -3), q8(H, I, 7), (5 / 128, -3 / 128, 7 / 128)),
             ((2, 2, 2), q2(I, H, 2.0 ** -6, -2.0 ** -5, 3), q2(I, H, 2.0 ** -5, -2.0 ** -4, 1),
              q2(H, I, 2.0 ** -6, 2.0 ** -6, 2), (1 / 64, -1 / 32, 3 / 64))]
    for fm, g, u, d, (a, b, c) in cases:
        rows = oracle.shared_expert(fm, g, u, d, x)
        assert rows.shape == (T, H)
        for t in range(T):
            gt, ut = a * S[t], b * S[t]
            want = c * I * (gt / (1 + math.exp(-gt))) * ut
            assert np.allclose(rows[t], want, rtol=1e-12, atol=0.0), (fm, t)


# ----------------------------------------------------------------- whole layer
@pytest.mark.parametrize("case", ["cfg1", "q2sm_bias"])
def test_layer_matches_brute_force(case):
    if case == "cfg1":
        wl = synth.make(1)
        rf = 0
    else:
        wl = synth.make(synth.custom(6, 256, 8, 64, 3, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1,
                                     bias="normal0.5"))
        rf = 1
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    got = oracle.layer(wl.x, rf, wl.router[0], wl.bias, wl.k, fm, wl.gate, wl.up, wl.down)
    ref = brute.layer(wl.x, rf, wl.router[0], wl.bias, wl.k, fm, wl.gate, wl.up, wl.down)
    assert np.all(ref["margin"] > 1e-4)
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.allclose(got["w"], ref["w"], rtol=2e-7, atol=0)
    assert np.allclose(got["out"], ref["out"], rtol=1e-6, atol=1e-7 * np.abs(ref["out"]).max())


# ----------------------------------------------------------------- ownership
def _small_share_case():
    cfg = synth.custom(12, 256, 16, 64, 4, gate_fmt=2, up_fmt=2, down_fmt=1, router_fmt=1,
                       bias="normal0.5", share=True)
    return synth.make(cfg)


def test_lpt_hand_example():
    assert oracle.place_lpt(np.array([5, 4, 3, 3, 2, 1]), 2).tolist() == [0, 1, 1, 0, 1, 0]
    # equal loads: experts in id order, each to the lighter share, ties to share 0
    assert oracle.place_lpt(np.array([1, 1, 1, 1]), 2).tolist() == [0, 1, 0, 1]


def _partials(wl, owner, n_shares, local_order=None, mutation=None):
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    outs = []
    for s in range(n_shares):
        g2l, l2g = oracle.share_tables(owner, s, local_order)
        r = oracle.layer(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k, fm,
                         wl.gate[l2g], wl.up[l2g], wl.down[l2g], g2l=g2l, mutation=mutation)
        outs.append(r["out"])
    return outs


def _full(wl):
    fm = (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)
    return oracle.layer(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k, fm, wl.gate, wl.up, wl.down)


@pytest.mark.parametrize("n_shares", [2, 4])
def test_partials_over_a_partition_sum_to_full(n_shares):
    wl = _small_share_case()
    full = _full(wl)["out"]
    owner = oracle.place_lpt(wl.load_hist, n_shares)
    parts = _partials(wl, owner, n_shares)
    total = np.sum([p.astype(np.float64) for p in parts], axis=0)
    assert np.max(np.abs(total - full)) <= 1e-6 * np.max(np.abs(full))
    # random (non-LPT) partition too
    owner_r = np.random.default_rng(n_shares).integers(0, n_shares, wl.E).astype(np.int32)
    parts = _partials(wl, owner_r, n_shares)
    total = np.sum([p.astype(np.float64) for p in parts], axis=0)
    assert np.max(np.abs(total - full)) <= 1e-6 * np.max(np.abs(full))


def test_every_slot_owned_exactly_once():
    wl = _small_share_case()
    ids, _, _ = oracle.route(wl.x, 1, wl.router[0], wl.bias, wl.k)
    for n in (2, 4):
        owner = oracle.place_lpt(wl.load_hist, n)
        hits = np.zeros(ids.shape, dtype=int)
        for s in range(n):
            g2l, _ = oracle.share_tables(owner, s)
            hits += g2l[ids] >= 0
        assert np.all(hits == 1)


def test_permuted_local_order_is_bit_identical():
    wl = _small_share_case()
    owner = oracle.place_lpt(wl.load_hist, 2)
    a = _partials(wl, owner, 2)
    b = _partials(wl, owner, 2, local_order=wl.local_perm)
    g2l_p, l2g_p = oracle.share_tables(owner, 0, wl.local_perm)
    assert np.any(l2g_p != np.arange(len(l2g_p)))             # local 0 != global 0 somewhere
    for pa, pb in zip(a, b):
        assert pa.tobytes() == pb.tobytes()


def test_shares_hold_several_experts_with_local_ne_global():
    # with one expert per share the local id is always 0 and a missing remap
    # goes unseen (arc PR #89: "ep4 survived the first mutation")
    wl = synth.make(5, T=1, experts=False)
    owner = oracle.place_lpt(wl.load_hist, 2)
    for s in range(2):
        g2l, l2g = oracle.share_tables(owner, s)
        assert len(l2g) == 128 and np.any(l2g != np.arange(128))
        g2l, l2g = oracle.share_tables(owner, s, wl.local_perm)
        assert np.any(l2g != np.sort(l2g))


@pytest.mark.parametrize("mutation", ["drop_remap", "never_mask", "combine_unmasked"])
def test_invariants_catch_planted_mistakes(mutation):
    """The three mutations of arc PR #89 ("The tests are the teeth"), planted in the
    oracle: each must break the partition-sum invariant or the permuted-placement
    invariant that the tests above assert."""
    wl = _small_share_case()
    full = _full(wl)["out"]
    owner = oracle.place_lpt(wl.load_hist, 2)
    parts = _partials(wl, owner, 2, local_order=wl.local_perm, mutation=mutation)
    total = np.sum([p.astype(np.float64) for p in parts], axis=0)
    sum_ok = np.max(np.abs(total - full)) <= 1e-6 * np.max(np.abs(full))
    plain = _partials(wl, owner, 2, mutation=mutation)
    perm_ok = all(p.tobytes() == q.tobytes() for p, q in zip(parts, plain))
    assert not (sum_ok and perm_ok)


def test_empty_batch():
    wl = synth.make(1, T=0)
    ids, w, z = oracle.route(wl.x.reshape(0, 256), 0, wl.router[0], None, 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)
    counts, offsets, slots = oracle.group(ids, 8)
    assert counts.sum() == 0 and offsets.tolist() == [0] * 9 and slots.size == 0



# ---- table routing ---------------------------------------------------------------------------
def _table_case():
    wl = synth.make(synth.custom(6, 256, 16, 128, 4, router_fmt=1, bias="zipf1.1", name="table"), experts=False)
    return wl, oracle.route(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k)


def test_route_table_with_top_k_rows_is_the_learned_route():
    """A table whose row t is token t's learned top k routes exactly as the top k does: the same
    ids in the same order, the same weights (the C oracle's top-k against the table path)."""
    wl, (ids, w, _) = _table_case()
    got_ids, got_w = oracle.route_table(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, np.arange(wl.T), ids)
    assert np.array_equal(got_ids, ids)
    np.testing.assert_allclose(got_w, w, rtol=1e-6, atol=0)


def test_route_table_follows_the_row_and_renormalises():
    """Reversing every table row reverses ids and weights; the weights of a row sum to 1; a token id
    picks its row, whatever the token's position."""
    wl, (ids, _, z) = _table_case()
    table = np.ascontiguousarray(ids[::-1, ::-1])      # row v = reversed top k of token T-1-v
    tok = np.arange(wl.T)[::-1].copy()
    got_ids, got_w = oracle.route_table(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, tok, table)
    assert np.array_equal(got_ids, ids[:, ::-1])
    np.testing.assert_allclose(got_w.sum(axis=1), 1.0, rtol=1e-6)
    # the largest logit of a row gets the largest weight
    for t in range(wl.T):
        assert int(got_ids[t, np.argmax(got_w[t])]) == int(got_ids[t, np.argmax(z[t, got_ids[t]])])
