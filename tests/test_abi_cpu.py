"""The C ABI without a GPU: exported symbols, host helpers, argument checks."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import quantized_moe_routed_amd as moe

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


@pytest.mark.parametrize("fmt,rows,cols", [(1, 3, 64), (2, 5, 96), (0, 2, 32)])
def test_pack_planar_is_the_documented_permutation(fmt, rows, cols):
    aos = synth.quant_matrices(11, 77, 2, rows, cols, fmt)
    codes, scales = moe.pack_planar(fmt, aos, 2, rows, cols)
    nb = cols // 32
    if fmt == 0:
        assert codes.tobytes() == aos.tobytes() and scales is None
        return
    bb = 34 if fmt == 1 else 12
    blocks = aos.reshape(-1, bb)
    hdr = 2 if fmt == 1 else 4
    assert scales.tobytes() == blocks[:, :hdr].tobytes()
    assert codes.tobytes() == blocks[:, hdr:].tobytes()
    # planar code bytes keep the definition's bit order: value i of a row in byte i/4
    if fmt == 2:
        deq = oracle.dequant_rows(2, aos.reshape(-1, nb * 12), cols)
        c = codes.reshape(-1, cols // 4)
        d = np.frombuffer(scales.tobytes(), np.float16).reshape(-1, nb, 2).astype(np.float64)
        q = np.stack([(c >> (2 * i)) & 3 for i in range(4)], -1).reshape(-1, nb, 32)
        assert np.array_equal(d[..., 0:1] * q + d[..., 1:2], deq.reshape(-1, nb, 32))


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


def test_bf16_forward_shape_and_format_limits():
    big = 1 << 30
    def call(H=256, I=128, gf=moe.W_Q2SM, df=moe.W_Q8_0):
        ex = moe.Experts(moe.qmat(gf, I, H, FAKE, FAKE), moe.qmat(gf, I, H, FAKE, FAKE),
                         moe.qmat(df, H, I, FAKE, FAKE), 8)
        moe.expert_forward(FAKE, moe.ACT_BF16, 4, H, I, 2, ex, None, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, big, 0)
    assert _status(lambda: call(H=160)) == moe.ERR_UNSUPPORTED          # H not a multiple of 64
    assert _status(lambda: call(I=96)) == moe.ERR_UNSUPPORTED           # I not a multiple of 64
    assert _status(lambda: call(gf=moe.W_Q8_0)) == moe.ERR_UNSUPPORTED  # MFMA path: Q2SM gate/up
    assert _status(lambda: call(df=moe.W_Q2SM)) == moe.ERR_UNSUPPORTED  # MFMA path: Q8_0 down
    a = moe.workspace_size(2048, 4096, 2048, 8, 256, 256, moe.ACT_BF16)
    assert a[2] >= 2048 * 8 * 2048 * 4 + 2048 * 128 * 4
