"""Oracle B: BF16 (or binary16) blocked emulation of the tiled
forward/backward (test infrastructure only).

It walks the one-pass tiled algorithm the pages describe -- blocks of keys,
an online ("safe") softmax with running row maximum and running row sum
(page 3, "What did Meta's study find": each block is rescaled and updated on
its own; page 2, "Mechanism 2: where the bias comes from": the row shift m of
safe softmax and the unnormalised output) -- row by row, with the kernel's
rounding sites, so that the rounding bias can be measured:

  * raw scores t = q.k rounded to FP32; the row maximum, the running shift and
    the running row sum are FP32;
  * the unnormalised probabilities P = 2^(t*c - M) (c = scale*log2 e, one
    fused multiply-add, one rounding) are FP32, and are cast to BF16
    (round-to-nearest-even) before the product with V;
  * the unnormalised output accumulates in FP32; O = bf16(O_bar * (1/l)).

The repeated-maximum fix (page 2, same section: detect whether the maximum
of a row of S occurs more than once, and if so shift m so that the exponent
at the maximum is strictly below 1).  The pages do not print the rule (the
listing announced there is missing), so this module takes the reading below;
its constants are parameters:

  * the count is the running count of the one-pass algorithm: when a block
    raises the running maximum the count restarts at that block's count of
    entries equal to it; when a block's maximum equals the running maximum
    its count is added; masked entries never count;
  * with R = m*c the running maximum in base-2 exponent units, the shift is
    M = R when the count is below 2 (or the fix is off) and otherwise
    M = R + delta(R) with delta(R) = max(|R|, delta_min) for |R| <= delta_max.
    For 0 < R <= delta_max that is M = 2R; for -delta_max <= R < 0 it is M = 0,
    so the largest probability becomes 2^-|R|: strictly below 1 (bf16 of it
    too: delta_min = 1/16 gives 0.957) and different from row to row;
  * above delta_max, |R| is folded down by whole multiples of FOLD = 32 into
    (delta_max - 32, delta_max].  An integer change of the exponent only
    rescales by a power of two, so the bf16 rounding of the largest
    probability -- which is what the fix changes -- stays that of 2^-|R|,
    while the largest probability stays at or above 2^-delta_max, far from
    FP32 underflow.  (A plain clamp at delta_max would give every such row the
    same power-of-two maximum 2^-64, whose bf16 rounding is exact: the fix
    would do nothing for them.)

For binary16 (``fmt="f16"``) the same rule folds |R| by whole units into
(0, 1] (``RULES["f16"]``): binary16's normal numbers end at 2^-14, so the
bf16 constants would let the largest probability 2^-|R| underflow once
|R| > 24.  A whole-unit fold rescales by a power of two only, so the rounding
of the largest probability stays that of 2^-|R|.

The size of the bias this rule removes, and the constants, are parity
unpinned: the pages give no number for them.

``no_round=True`` runs the identical recurrence in float64 with no casts; it
must then equal the exact oracle (``reference``) to ~1e-12 for any block size
and either variant, which pins the recurrence, the rescale and the shift logic.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

DELTA_MIN = 1.0 / 16.0   # base-2 exponent units
DELTA_MAX = 64.0
FOLD = 32.0

# binary16: the largest probability 2^-delta must stay far inside binary16's
# exponent range (normal numbers reach down to 2^-14 only), so |R| is folded
# by whole units into (0, 1]
F16_DELTA_MAX = 1.0
F16_FOLD = 1.0

RULES = {"bf16": (DELTA_MIN, DELTA_MAX, FOLD), "f16": (DELTA_MIN, F16_DELTA_MAX, F16_FOLD)}

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


# ----------------------------------------------------------------------------
# rounding primitives
# ----------------------------------------------------------------------------

def fl32(x):
    """Round float64 values to the nearest float32 (returned as float64)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """Round to the nearest bfloat16, ties to even (returned as float64).

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit, then
    clear the low 16 bits.  NaN stays NaN; +-inf stay; overflow rounds to inf.
    """
    with np.errstate(over="ignore"):
        x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(x32), np.nan, out)


def f16(x):
    """Round to the nearest IEEE binary16 value, ties to even (returned as
    float64): 11 significant bits, subnormals below 2^-14 with spacing 2^-24,
    overflow to inf from 65520 up.  The rounding is numpy's float32 -> float16
    conversion; the values rounded here are float32-exact, so going through
    float32 first adds no second rounding.
    """
    with np.errstate(over="ignore"):
        x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
        return x32.astype(np.float16).astype(np.float64)


FORMATS = {"bf16": bf16, "f16": f16}


def _rounders(no_round: bool, fmt: str = "bf16"):
    if no_round:
        ident = lambda x: np.asarray(x, dtype=np.float64)  # noqa: E731
        return ident, ident
    return fl32, FORMATS[fmt]


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------

def shift_rule(R: np.ndarray, tied: np.ndarray, stabilize: bool, delta_min: float,
               delta_max: float, no_round: bool, fold: float = FOLD) -> np.ndarray:
    """Shift M (base-2 units) from the running maximum R = m*c and the tie flag."""
    r32, _ = _rounders(no_round)
    if not stabilize:
        return R.copy()
    a = np.abs(R)
    with np.errstate(invalid="ignore"):
        over = np.where(a > delta_max, np.ceil((a - delta_max) / fold), 0.0)
    a = a - fold * over                       # exact in fp32: whole multiples of the fold
    delta = np.maximum(a, delta_min)
    shifted = r32(R + delta)
    return np.where(tied & np.isfinite(R), shifted, R)


def forward(q, k, v, scale: float, causal: bool, *, block: int = 64, stabilize: bool,
            no_round: bool = False, delta_min: Optional[float] = None, delta_max: Optional[float] = None,
            return_state: bool = False, fmt: str = "bf16", fold: Optional[float] = None):
    """Blocked forward of one or more heads.

    q, k, v: (..., N, d) arrays (values exact in ``fmt``, the 16-bit element
    type: "bf16", or "f16" for IEEE binary16, which replaces BF16 at every
    16-bit rounding site).  Returns (O, LSE) and,
    with ``return_state``, a dict with the final running count, the final
    shift M, whether each row was ever shifted, and the largest probability
    that entered the PV product at a shifted step (for the "< 1" check).
    """
    r32, rb16 = _rounders(no_round, fmt)
    rule = RULES[fmt]
    delta_min = rule[0] if delta_min is None else delta_min
    delta_max = rule[1] if delta_max is None else delta_max
    fold = rule[2] if fold is None else fold
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    N, d = q.shape[-2], q.shape[-1]
    Nk = k.shape[-2]
    q2 = q.reshape(-1, N, d)
    k2 = k.reshape(-1, Nk, d)
    v2 = v.reshape(-1, Nk, v.shape[-1])
    G = q2.shape[0]
    c = (scale * LOG2E) if no_round else float(np.float32(np.float32(scale) * np.float64(LOG2E)))

    m = np.full((G, N), -np.inf)
    cnt = np.zeros((G, N), dtype=np.int64)
    M = np.full((G, N), -np.inf)
    l = np.zeros((G, N))
    ob = np.zeros((G, N, v2.shape[-1]))
    ever = np.zeros((G, N), dtype=bool)
    pmax_shifted = np.full((G, N), -np.inf)
    rows = np.arange(N)[:, None]

    last_key = Nk
    for j0 in range(0, last_key, block):
        j1 = min(j0 + block, last_key)
        if causal and j0 > N - 1:
            break
        t = r32(q2 @ np.swapaxes(k2[:, j0:j1], -1, -2))            # (G, N, b)
        if causal:
            keys = np.arange(j0, j1)[None, :]
            t = np.where(keys > rows, -np.inf, t)
        bm = t.max(axis=-1)
        bc = ((t == bm[..., None]) & np.isfinite(t)).sum(axis=-1)
        up = bm > m
        same = (bm == m) & np.isfinite(bm)
        cnt = np.where(up, bc, np.where(same, cnt + bc, cnt))
        m = np.maximum(m, bm)
        R = r32(m * c)
        tied = cnt >= 2
        Mn = shift_rule(R, tied, stabilize, delta_min, delta_max, no_round, fold)
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(Mn), r32(np.exp2(r32(M - Mn))), 1.0)
        p = r32(np.exp2(r32(t * c - Mn[..., None])))                # masked -> exp2(-inf) = 0
        shifted_now = stabilize & tied & np.isfinite(Mn)
        ever |= shifted_now
        pm = np.where(shifted_now, p.max(axis=-1), -np.inf)
        pmax_shifted = np.maximum(pmax_shifted, rb16(pm))
        l = r32(r32(alpha * l) + p.sum(axis=-1))
        ob = r32(r32(alpha[..., None] * ob) + rb16(p) @ v2[:, j0:j1])
        M = Mn

    rinv = r32(1.0 / l)
    o = rb16(r32(ob * rinv[..., None]))
    lse = r32(r32(M + r32(np.log2(l))) * (LN2 if no_round else float(np.float32(LN2))))
    o = o.reshape(lead + (N, v2.shape[-1]))
    lse = lse.reshape(lead + (N,))
    if not return_state:
        return o, lse
    state = {"count": cnt.reshape(lead + (N,)), "shift": M.reshape(lead + (N,)),
             "ever_shifted": ever.reshape(lead + (N,)),
             "pmax_shifted_bf16": pmax_shifted.reshape(lead + (N,))}
    return o, lse, state


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

def backward(q, k, v, o, do, lse, scale: float, causal: bool, *, no_round: bool = False,
             fmt: str = "bf16"):
    """Backward from the saved LSE, with the kernel's rounding sites (16-bit
    sites in ``fmt``, as in ``forward``).

    D = rowsum(dO * O) uses the bf16 forward output O.  P = 2^(t*c - LSE*log2 e)
    is recomputed in FP32 (the shift plays no part: P depends only on LSE);
    bf16(P) enters dV; dS = P (dP - D) is FP32 and is cast to bf16 before the
    dK and dQ products; the accumulators are FP32 and the results bf16.
    """
    r32, rb16 = _rounders(no_round, fmt)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    N = q.shape[-2]
    if no_round:
        c, l2e = scale * LOG2E, LOG2E
        sc = scale
    else:
        c = float(np.float32(np.float32(scale) * np.float64(LOG2E)))
        l2e = float(np.float32(LOG2E))
        sc = float(np.float32(scale))
    t = r32(q @ np.swapaxes(k, -1, -2))
    lse2 = r32(lse * l2e)
    p = r32(np.exp2(r32(t * c - lse2[..., None])))
    if causal:
        p = np.where(np.triu(np.ones((N, k.shape[-2]), dtype=bool), 1), 0.0, p)
    dvec = r32((do * o).sum(axis=-1))
    dp = r32(do @ np.swapaxes(v, -1, -2))
    ds = r32(p * r32(dp - dvec[..., None]))
    dv = rb16(r32(np.swapaxes(rb16(p), -1, -2) @ do))
    dk = rb16(r32(sc * r32(np.swapaxes(rb16(ds), -1, -2) @ q)))
    dq = rb16(r32(sc * r32(rb16(ds) @ k)))
    return dq, dk, dv
