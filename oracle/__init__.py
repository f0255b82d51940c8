"""CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``quantized_moe_routed_amd``) and never imports it; the two meet only in the
seeded inputs of ``synth``.

The arithmetic lives in ``oracle.c`` (plain C loops, fp64 for the expert FFN
and the combine, the canonical fp32 order for router logits); this module adds
the placement and ownership bookkeeping in plain Python and marshals arrays.

Sources for each step (the three pages this layer is built from):

* ownership, global-to-local remap, partial sums that add up over a partition,
  LPT-balanced placement: aeonmindai/arc PR #89, section "Stage 1 -- EP=2";
* a permuted placement reproducing the unpermuted result, and the three
  mutations that the tests must catch: same page, "The tests are the teeth";
* a fixed-order, atomic-free accumulation of the routed down projection:
  TrevorS/ds4 PR #13, "Tested" (scheduling-dependent float atomics drift);
* routed gate/up/down quantisation roles: antirez/ds4 PR #754, "Supported
  paths and safety".

The routing formula (sigmoid scores, top-k with ties to the lower index,
renormalised weights) and the expert FFN (down(SiLU(gate x) * up x)) are
not written on the pages; they are the plain reading of the layer the pages
describe.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# MOE_ORACLE_LIB names another build of the same source (the sanitizer test builds one with
# -fsanitize=address,undefined); it is loaded as it is, without building
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")
_LIB_PATH = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

F32, Q8_0, Q2SM = 0, 1, 2
_BLOCK = {Q8_0: 34, Q2SM: 12}


def build(force: bool = False) -> str:
    if _LIB_OVERRIDE:
        return _LIB_PATH
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _L():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
            L.oracle_row_bytes.argtypes = [i32, i32]
            L.oracle_row_bytes.restype = i64
            L.oracle_dequant_row.argtypes = [i32, vp, i32, vp]
            L.oracle_router_logit.argtypes = [i32, vp, vp, i32, vp]
            L.oracle_router_logit.restype = f32
            L.oracle_route.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp]
            L.oracle_group.argtypes = [vp, i32, i32, i32, vp, vp, vp]
            L.oracle_expert.argtypes = [i32, vp, i32, vp, i32, vp, i32, i32, vp, vp]
            L.oracle_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
            _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def row_bytes(fmt: int, cols: int) -> int:
    return cols * 4 if fmt == F32 else (cols // 32) * _BLOCK[fmt]


# ---------------------------------------------------------------- dequantise
def dequant_rows(fmt: int, rows: np.ndarray, cols: int) -> np.ndarray:
    """Definition bytes [n, row_bytes] -> fp64 [n, cols], exactly."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1, row_bytes(fmt, cols))
    out = np.empty((rows.shape[0], cols), dtype=np.float64)
    L = _L()
    for r in range(rows.shape[0]):
        L.oracle_dequant_row(fmt, _p(rows[r]), cols, _p(out[r]))
    return out


# ---------------------------------------------------------------- route
def router_logit(fmt: int, wrow: np.ndarray, x: np.ndarray, bias_e: Optional[float] = None) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    wrow = np.ascontiguousarray(wrow, dtype=np.uint8)
    b = None if bias_e is None else np.array([bias_e], dtype=np.float32)
    return float(_L().oracle_router_logit(fmt, _p(wrow), _p(x), x.shape[-1], _p(b)))


def route(x: np.ndarray, router_fmt: int, router: np.ndarray, bias: Optional[np.ndarray], k: int):
    """x fp32 [T,H]; router definition bytes [E, row_bytes].  Returns ids [T,k] int32,
    w [T,k] fp32 and the logits z [T,E] fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    router = np.ascontiguousarray(router, dtype=np.uint8).reshape(-1, row_bytes(router_fmt, H))
    E = router.shape[0]
    assert 1 <= k <= E
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    z = np.empty((T, E), dtype=np.float32)
    if T:
        _L().oracle_route(_p(x), T, H, E, router_fmt, _p(router), _p(b), k, _p(ids), _p(w), _p(z))
    return ids, w, z


def route_table(x: np.ndarray, router_fmt: int, router: np.ndarray, bias: Optional[np.ndarray],
                token_ids: np.ndarray, table: np.ndarray):
    """Table routing (aeonmindai/arc PR #89, "Stage 0": the first layers of the model route by a
    fixed token-id table).  The experts of token t are row token_ids[t] of table [V, k], in the
    row's order.  The page gives no weight rule; the reading is the learned routes' rule:
    sigmoid of each expert's logit (the same logits as route(), bias included), renormalised over
    the row, in fp64, rounded to fp32.  Returns ids [T,k] int32 and w [T,k] fp32."""
    table = np.asarray(table, dtype=np.int32)
    k = table.shape[1]
    _, _, z = route(x, router_fmt, router, bias, 1)
    ids = table[np.asarray(token_ids, dtype=np.int64)]
    w = np.empty(ids.shape, dtype=np.float32)
    for t in range(ids.shape[0]):
        s = [1.0 / (1.0 + np.exp(-float(z[t, e]))) for e in ids[t]]
        tot = sum(s)
        for j in range(k):
            w[t, j] = np.float32(s[j] / tot)
    return ids.astype(np.int32), w


def shared_expert(fmts: Sequence[int], gate: np.ndarray, up: np.ndarray, down: np.ndarray,
                  x: np.ndarray) -> np.ndarray:
    """The shared expert's rows [T, H] (fp64): expert() of the one-expert stack on every token (the
    pages name a shared expert beside the routed ones, antirez/ds4 PR #754, "Supported paths and
    safety"; the caller adds it to the routed output in fp32)."""
    return np.stack([expert(fmts, gate[0], up[0], down[0], x[t]) for t in range(x.shape[0])])


# ---------------------------------------------------------------- group
def group(ids: np.ndarray, E: int):
    """Stable grouping of slots s = t*k + j by expert id."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    slot_list = np.empty(T * k, dtype=np.int32)
    _L().oracle_group(_p(ids), T, k, E, _p(counts), _p(offsets), _p(slot_list))
    return counts, offsets, slot_list


# ---------------------------------------------------------------- experts
def expert(fmts: Sequence[int], gate: np.ndarray, up: np.ndarray, down: np.ndarray,
           x: np.ndarray) -> np.ndarray:
    """One expert on one token in fp64.  gate/up: [I, row_bytes(H)], down: [H, row_bytes(I)]."""
    I = gate.shape[0]
    H = down.shape[0]
    xd = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(H, dtype=np.float64)
    g, u, d = (np.ascontiguousarray(a, dtype=np.uint8) for a in (gate, up, down))
    _L().oracle_expert(fmts[0], _p(g), fmts[1], _p(u), fmts[2], _p(d), H, I, _p(xd), _p(y))
    return y


def combine(y_slot: np.ndarray, w: np.ndarray, ids: np.ndarray, g2l: Optional[np.ndarray]) -> np.ndarray:
    """out[t] = sum over owned j ascending of w[t,j] * y_slot[t*k+j] (fp64, one rounding)."""
    T, k = ids.shape
    H = y_slot.shape[1]
    y = np.ascontiguousarray(y_slot, dtype=np.float64)
    out = np.empty((T, H), dtype=np.float32)
    g = None if g2l is None else np.ascontiguousarray(g2l, dtype=np.int32)
    _L().oracle_combine(_p(y), _p(np.ascontiguousarray(w, np.float32)),
                        _p(np.ascontiguousarray(ids, np.int32)), _p(g), T, k, H, _p(out))
    return out


# ---------------------------------------------------------------- placement
def place_lpt(load: np.ndarray, n_shares: int) -> np.ndarray:
    """LPT-balanced placement (arc PR #89, Stage 1 names contiguous / explicit /
    LPT-balanced placements).  Experts in order of load descending, ties to the
    lower id, each to the least-loaded share that still has room (E / n_shares
    experts per share), ties to the lower share id.  Returns owner[E]."""
    load = [int(v) for v in load]
    E = len(load)
    assert n_shares >= 1 and E % n_shares == 0
    cap = E // n_shares
    order = sorted(range(E), key=lambda e: (-load[e], e))
    share_load = [0] * n_shares
    share_n = [0] * n_shares
    owner = np.empty(E, dtype=np.int32)
    for e in order:
        best = None
        for s in range(n_shares):
            if share_n[s] >= cap:
                continue
            if best is None or share_load[s] < share_load[best]:
                best = s
        owner[e] = best
        share_load[best] += load[e]
        share_n[best] += 1
    return owner


def share_tables(owner: np.ndarray, share: int, local_order: Optional[np.ndarray] = None):
    """Global->local table g2l [E] (-1 = unowned) and l2g [E_local] for one share.
    Local ids follow ascending global id, or ascending local_order[e] when given
    (a permuted placement, where local 0 is not global 0)."""
    E = len(owner)
    owned = [e for e in range(E) if owner[e] == share]
    if local_order is not None:
        owned.sort(key=lambda e: (int(local_order[e]), e))
    l2g = np.array(owned, dtype=np.int32)
    g2l = np.full(E, -1, dtype=np.int32)
    for l, e in enumerate(owned):
        g2l[e] = l
    return g2l, l2g


# ---------------------------------------------------------------- the layer
def forward_slots(fmts, gate, up, down, x: np.ndarray, ids: np.ndarray, slots: Sequence[int],
                  g2l: Optional[np.ndarray] = None, mutation: Optional[str] = None):
    """y_slot rows (fp64) for the given slots s = t*k + j.

    gate/up/down are the expert stacks the caller owns: indexed by global id
    when g2l is None, else by local id (the owned share's stack).  Unowned
    slots get no row (None).  `mutation` plants one of the three mistakes of
    arc PR #89 ("The tests are the teeth") so that tests can show they catch
    it: "drop_remap" indexes the local stack with the global id; "never_mask"
    computes unowned slots too."""
    k = ids.shape[1]
    E_local = gate.shape[0]
    rows = {}
    for s in slots:
        t, j = divmod(int(s), k)
        g = int(ids[t, j])
        if g2l is None:
            e = g
        else:
            loc = int(g2l[g])
            if mutation == "drop_remap":
                loc = g % E_local if loc >= 0 else loc
            if loc < 0:
                if mutation != "never_mask":
                    continue
                loc = g % E_local
            e = loc
        rows[int(s)] = expert(fmts, gate[e], up[e], down[e], x[t])
    return rows


def layer(x: np.ndarray, router_fmt: int, router: np.ndarray, bias, k: int, fmts, gate, up, down,
          g2l: Optional[np.ndarray] = None, tokens: Optional[Sequence[int]] = None,
          mutation: Optional[str] = None):
    """The whole layer (or one share's partial when g2l is given) for the listed tokens.

    Returns dict with ids, w (for those tokens), y (fp64 [n_tok*k, H], NaN rows for
    unowned slots) and out fp32 [n_tok, H]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    tok = list(range(T)) if tokens is None else [int(t) for t in tokens]
    xs = x[tok]
    ids, w, z = route(xs, router_fmt, router, bias, k)
    slots = range(len(tok) * k)
    rows = forward_slots(fmts, gate, up, down, xs, ids, slots, g2l, mutation)
    y = np.full((len(tok) * k, H), np.nan, dtype=np.float64)
    for s, r in rows.items():
        y[s] = r
    mask_g2l = g2l
    if mutation == "combine_unmasked" or mutation == "never_mask":
        mask_g2l = None
        if mutation == "combine_unmasked":
            y = np.where(np.isnan(y), 0.0, y)
            # unowned slots keep their routing weight and pick up the local
            # expert at index 0, as a combine that ignores the mask would
            for s in range(len(tok) * k):
                if g2l is not None and g2l[ids[s // k, s % k]] < 0:
                    y[s] = expert(fmts, gate[0], up[0], down[0], xs[s // k])
    out = combine(y, w, ids, mask_g2l)
    return dict(ids=ids, w=w, z=z, y=y, out=out, tokens=tok)
