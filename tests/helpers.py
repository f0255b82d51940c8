"""Shared test helpers: tolerance check and oracle expectations for a workload."""
from __future__ import annotations

import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402

# Output tolerance for floating-point results: max|d| <= 2e-3 max|ref| and
# ||d||_2 / ||ref||_2 <= 1e-4 (both must hold).
MAX_ABS_FRAC = 2e-3
REL_L2 = 1e-4


def close_report(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    mref = float(np.max(np.abs(ref))) if ref.size else 0.0
    nref = float(np.linalg.norm(ref))
    mabs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    return mabs, mref, rel


def assert_close(got, ref, what=""):
    mabs, mref, rel = close_report(got, ref)
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite values"
    assert mabs <= MAX_ABS_FRAC * mref + 1e-30, f"{what}: max|d| = {mabs:.3e} > {MAX_ABS_FRAC} * {mref:.3e}"
    assert rel <= REL_L2, f"{what}: rel-L2 = {rel:.3e} > {REL_L2}"


def sha(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def fmts(wl):
    return (wl.cfg.gate_fmt, wl.cfg.up_fmt, wl.cfg.down_fmt)


def oracle_expect(wl, tokens=None, l2g=None, g2l=None):
    """Oracle ids/w/y/out for the listed tokens (all by default).  With l2g/g2l,
    the partial of the share that owns l2g (local-indexed stack)."""
    if l2g is None:
        gate, up, down = wl.gate, wl.up, wl.down
    else:
        gate, up, down = wl.gate[l2g], wl.up[l2g], wl.down[l2g]
    return oracle.layer(wl.x, wl.cfg.router_fmt, wl.router[0], wl.bias, wl.k, fmts(wl), gate, up, down,
                        g2l=g2l, tokens=tokens)


def decode_planar(fmt, codes, scales, n, rows, cols):
    """Values of n planar matrices, decoded from the row-group layout as include/moe.h documents it."""
    nb = cols // 32
    if fmt == 0:
        return codes.view(np.float32).astype(np.float64).reshape(n * rows, cols)
    rg = (rows + 15) // 16
    out = np.zeros((n, rg * 16, cols))
    if fmt == 1:
        nu = (nb + 1) // 2
        c = codes.reshape(n, rg, nu, 16, 64)
        d = scales.view(np.float16).astype(np.float64).reshape(n, rg, nu, 16, 2)
        for b in range(nb):
            u, h = b // 2, b % 2
            for g in range(4):
                q = c[:, :, u, :, 16 * g + 8 * h:16 * g + 8 * h + 8].view(np.int8).astype(np.float64)
                out[:, :, 32 * b + 8 * g:32 * b + 8 * g + 8] = (d[:, :, u, :, h:h + 1] * q).reshape(n, rg * 16, 8)
    else:
        nu = (nb + 7) // 8
        c = codes.reshape(n, rg, nu, 16, 64)
        sc = scales.view(np.float16).astype(np.float64).reshape(n, rg, nu, 2, 16, 8)   # d rows, then m rows
        for b in range(nb):
            u, k = b // 8, b % 8
            i, h = k // 2, k % 2
            d = sc[:, :, u, 0, :, k].reshape(n, rg * 16)
            m = sc[:, :, u, 1, :, k].reshape(n, rg * 16)
            for g in range(4):
                lo_byte = c[:, :, u, :, 16 * g + 4 * i + h].reshape(n, rg * 16)       # definition byte 2g
                hi_byte = c[:, :, u, :, 16 * g + 4 * i + 2 + h].reshape(n, rg * 16)   # definition byte 2g+1
                for s in range(4):
                    out[:, :, 32 * b + 8 * g + s] = d * ((lo_byte >> (2 * s)) & 3) + m
                    out[:, :, 32 * b + 8 * g + 4 + s] = d * ((hi_byte >> (2 * s)) & 3) + m
    # rows that pad the last group hold zeros
    assert not out[:, rows:, :].any()
    return out[:, :rows, :].reshape(n * rows, cols)
