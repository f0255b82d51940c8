"""The C ABI without a GPU: exported symbols, host helpers, argument checks."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import quantized_moe_routed_amd as moe
from helpers import decode_planar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(moe.lib, n), n
        assert n in moe.EXPORTS


def test_version():
    assert moe.version().startswith("moe-gfx950")


def test_large_tile_threshold_by_batch_size():
    """Small tiles only up to 32 tokens; up to 255 tokens only experts of more than 4 small tiles
    take large ones; from 256 tokens experts of 12 or more slots do."""
    assert [moe.large_tile_min(T) for T in (0, 1, 8, 9, 32)] == [0] * 5
    assert [moe.large_tile_min(T) for T in (33, 128, 255)] == [33] * 3
    assert [moe.large_tile_min(T) for T in (256, 2048, 1 << 20)] == [12] * 3


@pytest.mark.parametrize("fmt,rows,cols", [(1, 3, 64), (1, 2, 160), (1, 37, 96), (2, 5, 96), (2, 3, 2080),
                                           (2, 2, 256), (2, 33, 320), (0, 2, 32)])
def test_pack_planar_is_the_documented_unit_layout(fmt, rows, cols):
    aos = synth.quant_matrices(11, 77, 2, rows, cols, fmt)
    codes, scales = moe.pack_planar(fmt, aos, 2, rows, cols)
    cb, sb = moe.planar_bytes(fmt, rows, cols)
    assert codes.size == 2 * cb and (scales is None) == (sb == 0)
    got = decode_planar(fmt, codes, scales, 2, rows, cols)
    ref = oracle.dequant_rows(fmt, aos.reshape(2 * rows, -1), cols)
    assert np.array_equal(got, ref)
    nb = cols // 32
    rg = (rows + 15) // 16
    if fmt == 1 and nb % 2:                  # scale and code padding of a row's last unit is zero
        nu = (nb + 1) // 2
        assert not scales.view(np.uint16).reshape(2, rg, nu, 16, 2)[:, :, -1, :, 1].any()
        c = codes.reshape(2, rg, nu, 16, 4, 16)
        assert not c[:, :, -1, :, :, 8:].any()
    if fmt == 2 and nb % 8:                  # padding blocks of a row's last unit are zero, codes and scales
        nu = (nb + 7) // 8
        sc = scales.view(np.uint16).reshape(2, rg, nu, 2, 16, 8)
        assert not sc[:, :, -1, :, :, nb % 8:].any()
        c = codes.reshape(2, rg, nu, 16, 64)
        for k in range(nb % 8, 8):
            i, h = k // 2, k % 2
            for g in range(4):
                assert not c[:, :, -1, :, 16 * g + 4 * i + h].any()
                assert not c[:, :, -1, :, 16 * g + 4 * i + 2 + h].any()


def test_lpt_matches_oracle():
    rng = np.random.default_rng(0)
    for E, n in [(256, 2), (16, 4), (12, 3), (8, 8)]:
        load = rng.integers(0, 50, E)
        assert np.array_equal(moe.place_lpt(load, n), oracle.place_lpt(load, n))
    wl = synth.make(5, T=1, experts=False)
    owner = moe.place_lpt(wl.load_hist, 2)
    assert np.array_equal(owner, oracle.place_lpt(wl.load_hist, 2))
    for s in range(2):
        for order in (None, wl.local_perm):
            g2l, l2g = moe.share_tables(owner, s, order)
            og2l, ol2g = oracle.share_tables(owner, s, order)
            assert np.array_equal(g2l, og2l) and np.array_equal(l2g, ol2g)
            moe.plan_check(g2l, len(l2g))


def test_plan_check_rejects_bad_tables():
    with pytest.raises(moe.MoeError) as e:
        moe.plan_check(np.array([0, 0, -1], np.int32), 1)
    assert e.value.status == moe.ERR_ARG
    with pytest.raises(moe.MoeError):
        moe.plan_check(np.array([0, 1, -1], np.int32), 3)       # E_local disagrees with owned count
    with pytest.raises(moe.MoeError):
        moe.plan_check(np.array([0, 5, -1], np.int32), 2)       # local id out of range
    with pytest.raises(moe.MoeError):
        moe.plan_check(np.array([0, -2, 1], np.int32), 2)
    moe.plan_check(np.array([1, -1, 0], np.int32), 2)


def test_workspace_sizes_grow_with_tokens():
    a = moe.workspace_size(1, 4096, 2048, 8, 256, 256, moe.ACT_F32)
    b = moe.workspace_size(32, 4096, 2048, 8, 256, 256, moe.ACT_F32)
    assert all(x <= y for x, y in zip(a, b))
    assert b[2] >= 32 * 8 * 2048 * 4


# ---- argument errors are reported before anything touches a device ---------------
FAKE = 1 << 20   # a non-NULL, 16-byte aligned address that is never dereferenced


def _router(fmt=moe.W_Q8_0, rows=8, cols=256):
    return moe.qmat(fmt, rows, cols, FAKE, FAKE)


def _status(fn, *args):
    with pytest.raises(moe.MoeError) as e:
        fn(*args)
    return e.value.status


def test_route_argument_errors():
    r = _router()
    call = lambda **kw: moe.route(kw.get("x", FAKE), kw.get("xt", 0), kw.get("T", 4), kw.get("H", 256),
                                  kw.get("router", r), None, kw.get("k", 2), FAKE, FAKE, FAKE,
                                  kw.get("ws", 1 << 20), 0)
    assert _status(lambda: call(k=9)) == moe.ERR_ARG                # k > E
    assert _status(lambda: call(k=0)) == moe.ERR_ARG
    assert _status(lambda: call(H=100)) == moe.ERR_ARG              # not a multiple of 32
    assert _status(lambda: call(T=-1)) == moe.ERR_ARG
    assert _status(lambda: call(xt=7)) == moe.ERR_ARG
    assert _status(lambda: call(x=None)) == moe.ERR_ARG
    assert _status(lambda: call(ws=16)) == moe.ERR_WORKSPACE
    assert _status(lambda: call(router=_router(fmt=moe.W_Q2SM))) == moe.ERR_UNSUPPORTED
    assert _status(lambda: call(router=_router(rows=2000))) == moe.ERR_UNSUPPORTED
    assert _status(lambda: call(router=_router(cols=128))) == moe.ERR_ARG      # shape disagrees with H
    assert _status(lambda: call(x=FAKE + 4)) == moe.ERR_ARG          # misaligned
    assert "k = 9" in _msg(lambda: call(k=9))
    call(T=0)                                                        # T = 0: a successful no-op


def _msg(fn):
    try:
        fn()
    except moe.MoeError as e:
        return str(e)
    return ""


def _experts(E_local=8, H=256, I=128, gf=moe.W_Q8_0, df=moe.W_Q8_0, n=None):
    return moe.Experts(moe.qmat(gf, I, H, FAKE, FAKE), moe.qmat(gf, I, H, FAKE, FAKE),
                       moe.qmat(df, H, I, FAKE, FAKE), E_local if n is None else n)


def test_forward_argument_errors():
    big = 1 << 30
    def call(**kw):
        ex = kw.get("ex", _experts())
        moe.expert_forward(FAKE, kw.get("xt", 0), kw.get("T", 4), kw.get("H", 256), kw.get("I", 128),
                           kw.get("k", 2), ex, kw.get("g2l", None), kw.get("E", 8), kw.get("E_local", 8),
                           FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("ws", big), 0)
    assert _status(lambda: call(E_local=4)) == moe.ERR_ARG                       # E_local != stack size
    assert _status(lambda: call(ex=_experts(4), E_local=4)) == moe.ERR_ARG       # partial stack, no g2l
    assert _status(lambda: call(ex=_experts(gf=moe.W_F32))) == moe.ERR_UNSUPPORTED
    assert _status(lambda: call(ex=_experts(I=64))) == moe.ERR_ARG               # shape disagrees
    assert _status(lambda: call(H=16384, ex=_experts(H=16384))) == moe.ERR_UNSUPPORTED
    assert _status(lambda: call(ws=64)) == moe.ERR_WORKSPACE
    assert _status(lambda: call(k=9)) == moe.ERR_ARG
    call(T=0)


def test_group_and_combine_argument_errors():
    assert _status(lambda: moe.group_tokens(FAKE, 4, 2, 2000, FAKE, FAKE, FAKE, stream=0)) == moe.ERR_UNSUPPORTED
    assert _status(lambda: moe.group_tokens(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, stream=0)) == moe.ERR_ARG
    assert _status(lambda: moe.group_tokens(FAKE, 4, 2, 8, None, FAKE, FAKE, stream=0)) == moe.ERR_ARG
    assert _status(lambda: moe.combine(FAKE, FAKE, FAKE, None, 4, 2, 6, 8, FAKE, stream=0)) == moe.ERR_ARG
    assert _status(lambda: moe.combine(None, FAKE, FAKE, None, 4, 2, 256, 8, FAKE, stream=0)) == moe.ERR_ARG
    moe.combine(FAKE, FAKE, FAKE, None, 0, 2, 256, 8, FAKE, stream=0)


def test_bf16_forward_format_limits():
    big = 1 << 30
    def call(gf=moe.W_Q2SM, df=moe.W_Q8_0, H=256, I=128):
        ex = moe.Experts(moe.qmat(gf, I, H, FAKE, FAKE), moe.qmat(gf, I, H, FAKE, FAKE),
                         moe.qmat(df, H, I, FAKE, FAKE), 8)
        moe.expert_forward(FAKE, moe.ACT_BF16, 4, H, I, 2, ex, None, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, big, 0)
    assert _status(lambda: call(gf=moe.W_F32)) == moe.ERR_UNSUPPORTED
    assert _status(lambda: call(df=moe.W_F32)) == moe.ERR_UNSUPPORTED
    a = moe.workspace_size(2048, 4096, 2048, 8, 256, 256, moe.ACT_BF16)
    f = moe.workspace_size(2048, 4096, 2048, 8, 256, 256, moe.ACT_F32)
    assert a[2] >= 2048 * 8 * 2048 * 4 + 2048 * 4096 * 2
    # fp32 activations add the lo plane and, their staging of 8 rows not fitting two workgroups per
    # compute unit at H = 4096, take small tiles of 4 slots.  Large tiles take every expert of 12
    # slots or more (T = 2048), so an expert has at most ceil(11 / 4) = 3 small tiles of 4 slots
    # against ceil(11 / 8) = 2 of 8: 256 more tiles of 16 + 32 bytes.  The down projection, whose
    # staging of 8 rows does fit (K = I = 2048), keeps a list of its own small tiles of 8 slots: at
    # most 2 per expert, 512 tiles of 16 bytes, and its count (one 256-byte aligned slot)
    assert moe.large_tile_min(2048) == 12
    assert f[2] == a[2] + 2048 * 4096 * 2 + 256 * (3 - 2) * (16 + 32) + 512 * 16 + 256


def test_build_scan_flags_dpp_operand_written_too_late():
    """The library build rejects a DPP instruction whose operand a vector instruction wrote fewer
    than two wait states before (s_nop N counts N + 1)."""
    from quantized_moe_routed_amd.build import _dpp_hazards
    bad = "v_cvt_f32_i32_e32 v5, v1\n\tv_fmac_f32_dpp v3, v5, v4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
    assert len(_dpp_hazards(bad)) == 1
    one = "v_cvt_f32_i32_e32 v5, v1\n\ts_nop 0\n\tv_fmac_f32_dpp v3, v5, v4 row_newbcast:0\n"
    assert len(_dpp_hazards(one)) == 1
    ok = "v_cvt_f32_i32_e32 v5, v1\n\ts_nop 1\n\tv_fmac_f32_dpp v3, v5, v4 row_newbcast:0\n"
    assert _dpp_hazards(ok) == []
    other = "v_cvt_f32_i32_e32 v6, v1\n\tv_fmac_f32_dpp v3, v5, v4 row_newbcast:0\n"
    assert _dpp_hazards(other) == []



def test_table_check_and_route_table_argument_errors():
    moe.table_check(np.array([[0, 3], [2, 1], [3, 0]], np.int32), 4)
    for bad in ([[0, 4], [1, 2]], [[0, -1], [1, 2]], [[1, 1], [0, 2]]):
        with pytest.raises(moe.MoeError) as e:
            moe.table_check(np.array(bad, np.int32), 4)
        assert e.value.status == moe.ERR_ARG
    r = _router()
    call = lambda **kw: moe.route_table(FAKE, 0, 4, 256, r, None, kw.get("tok", FAKE), kw.get("table", FAKE),
                                        kw.get("V", 16), 2, FAKE, FAKE, FAKE, 1 << 20, 0)
    assert _status(lambda: call(table=None)) == moe.ERR_ARG
    assert _status(lambda: call(tok=None)) == moe.ERR_ARG
    assert _status(lambda: call(V=0)) == moe.ERR_ARG



def test_shared_expert_argument_errors():
    assert moe.shared_expert_workspace(4, 256, 128, moe.ACT_F32) > 4 * 256 * 4
    ex = lambda n: moe.Experts(moe.qmat(moe.W_Q8_0, 128, 256, FAKE, FAKE), moe.qmat(moe.W_Q8_0, 128, 256, FAKE, FAKE),
                               moe.qmat(moe.W_Q8_0, 256, 128, FAKE, FAKE), n)
    call = lambda n=1, ws=1 << 24: moe.shared_expert_forward(FAKE, moe.ACT_F32, 4, 256, 128, ex(n), FAKE, FAKE, ws, 0)
    assert _status(lambda: call(n=2)) == moe.ERR_ARG
    assert _status(lambda: call(ws=64)) == moe.ERR_WORKSPACE
