"""Brute-force evaluation of the layer in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

Independent of ``oracle.c``: it decodes the blocks with its own vectorised
numpy code, evaluates EVERY expert on EVERY token, scores with an fp64 matrix
product (no canonical order), and only then selects and combines.  Used on
small inputs to pin the oracle: expert ids agree whenever the k-th/(k+1)-th
logit margin is clear of fp32 rounding, and outputs agree to fp64 rounding.
"""
from __future__ import annotations

import numpy as np


def _half(u16: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode(fmt: int, rows: np.ndarray, cols: int) -> np.ndarray:
    """Definition bytes [..., row_bytes] -> fp64 [..., cols]."""
    lead = rows.shape[:-1]
    nb = cols // 32
    if fmt == 0:
        return np.ascontiguousarray(rows).view(np.float32).astype(np.float64).reshape(*lead, cols)
    if fmt == 1:
        blk = rows.reshape(*lead, nb, 34)
        d = _half(blk[..., 0:2].copy().view(np.uint16)[..., 0])
        q = blk[..., 2:34].copy().view(np.int8).astype(np.float64)
        return (d[..., None] * q).reshape(*lead, cols)
    blk = rows.reshape(*lead, nb, 12)
    d = _half(blk[..., 0:2].copy().view(np.uint16)[..., 0])
    m = _half(blk[..., 2:4].copy().view(np.uint16)[..., 0])
    qs = blk[..., 4:12].astype(np.uint8)
    codes = np.stack([(qs >> (2 * i)) & 3 for i in range(4)], axis=-1)   # [..., 8 bytes, 4]
    codes = codes.reshape(*lead, nb, 32).astype(np.float64)
    return (d[..., None] * codes + m[..., None]).reshape(*lead, cols)


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def all_experts(fmts, gate, up, down, x: np.ndarray) -> np.ndarray:
    """Y[e, t, :] = expert e applied to token t, fp64."""
    E, I = gate.shape[0], gate.shape[1]
    H = down.shape[1]
    xd = x.astype(np.float64)
    Y = np.empty((E, x.shape[0], H))
    for e in range(E):
        G = decode(fmts[0], gate[e], H)
        U = decode(fmts[1], up[e], H)
        D = decode(fmts[2], down[e], I)
        h = silu(xd @ G.T) * (xd @ U.T)
        Y[e] = h @ D.T
    return Y


def layer(x, router_fmt, router, bias, k, fmts, gate, up, down, owned=None):
    """Full layer by brute force.  owned: optional bool [E] mask for a partial."""
    T, H = x.shape
    E = gate.shape[0]
    Wr = decode(router_fmt, router.reshape(E, -1), H)
    z = x.astype(np.float64) @ Wr.T
    if bias is not None:
        z = z + bias.astype(np.float64)[None, :]
    ids = np.empty((T, k), dtype=np.int64)
    margin = np.empty(T)
    for t in range(T):
        order = np.lexsort((np.arange(E), -z[t]))
        ids[t] = order[:k]
        margin[t] = z[t, order[k - 1]] - z[t, order[k]] if k < E else np.inf
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(z, ids, 1)))
    w = s / s.sum(1, keepdims=True)
    Y = all_experts(fmts, gate, up, down, x)
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if owned is None or owned[ids[t, j]]:
                out[t] += w[t, j] * Y[ids[t, j], t]
    return dict(ids=ids, w=w, z=z, margin=margin, out=out, Y=Y)
