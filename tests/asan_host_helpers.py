"""The host helpers of libmoe (host.cpp) built alone with the host compiler's address and
undefined-behaviour sanitizers, loaded from MOE_HOST_LIB: the planar packer against an independent
decoder and the oracle's dequantisation, LPT placement and share tables against the oracle, and
the load-time checks' error paths.  Run by tests/test_sanitizers.py, not collected on its own."""
import ctypes
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import decode_planar

_path = os.environ.get("MOE_HOST_LIB")
pytestmark = pytest.mark.skipif(not _path, reason="MOE_HOST_LIB (a sanitized host-helper build) is not set")

if _path:
    L = ctypes.CDLL(_path)
    i32, vp, psz = ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_planar_bytes.argtypes = [i32, i32, i32, psz, psz]
    L.moe_pack_planar.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    L.moe_place_lpt.argtypes = [vp, i32, i32, vp]
    L.moe_share_tables.argtypes = [vp, i32, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_int32)]
    L.moe_plan_check.argtypes = [vp, i32, i32]
    L.moe_table_check.argtypes = [vp, i32, i32, i32]


def _p(a):
    return None if a is None else a.ctypes.data


def planar_bytes(fmt, rows, cols):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_planar_bytes(fmt, rows, cols, ctypes.byref(c), ctypes.byref(s)) == 0
    return c.value, s.value


@pytest.mark.parametrize("fmt,rows,cols", [(1, 3, 64), (1, 37, 96), (2, 5, 96), (2, 3, 2080), (2, 33, 320),
                                           (0, 2, 32)])
def test_pack_planar(fmt, rows, cols):
    aos = synth.quant_matrices(11, 77, 2, rows, cols, fmt)
    cb, sb = planar_bytes(fmt, rows, cols)
    codes = np.full(2 * cb, 0xAB, np.uint8)
    scales = np.full(max(2 * sb, 1), 0xAB, np.uint8)
    assert L.moe_pack_planar(fmt, 2, rows, cols, _p(aos), _p(codes), _p(scales) if sb else None) == 0
    got = decode_planar(fmt, codes, scales[: 2 * sb] if sb else None, 2, rows, cols)
    assert np.array_equal(got, oracle.dequant_rows(fmt, aos.reshape(2 * rows, -1), cols))


def test_lpt_and_share_tables():
    rng = np.random.default_rng(0)
    for E, n in [(256, 2), (16, 4), (12, 3), (8, 8)]:
        load = rng.integers(0, 50, E).astype(np.int64)
        owner = np.empty(E, np.int32)
        assert L.moe_place_lpt(_p(load), E, n, _p(owner)) == 0
        assert np.array_equal(owner, oracle.place_lpt(load, n))
        order = rng.permutation(E).astype(np.int32)
        for s in range(n):
            g2l, l2g, el = np.empty(E, np.int32), np.empty(E, np.int32), ctypes.c_int32()
            assert L.moe_share_tables(_p(owner), E, s, _p(order), _p(g2l), _p(l2g), ctypes.byref(el)) == 0
            og2l, ol2g = oracle.share_tables(owner, s, order)
            assert np.array_equal(g2l, og2l) and np.array_equal(l2g[: el.value], ol2g)
            assert L.moe_plan_check(_p(g2l), E, el.value) == 0


def test_error_paths():
    bad = [np.array([0, 0, -1], np.int32), np.array([0, 5, -1], np.int32), np.array([0, -2, 1], np.int32)]
    for t in bad:
        assert L.moe_plan_check(_p(t), 3, 2) != 0 and L.moe_last_error()
    tab = np.array([[0, 1], [2, 2]], np.int32)
    assert L.moe_table_check(_p(tab), 2, 2, 4) != 0 and b"twice" in L.moe_last_error()
    tab = np.array([[0, 9]], np.int32)
    assert L.moe_table_check(_p(tab), 1, 2, 4) != 0
    assert L.moe_planar_bytes(1, 3, 33, None, None) != 0
    assert L.moe_pack_planar(7, 1, 1, 32, _p(np.zeros(64, np.uint8)), _p(np.zeros(64, np.uint8)),
                             _p(np.zeros(64, np.uint8))) != 0
    load = np.ones(6, np.int64)
    assert L.moe_place_lpt(_p(load), 6, 4, _p(np.empty(6, np.int32))) != 0   # E not a multiple of shares
