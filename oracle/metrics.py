"""Error statistics against the exact oracle (test infrastructure only).

The pages report a "maximum relative error" of the attention output against a
high-precision baseline (page 3, "What did Meta's study find": about 1e-1 for
FlashAttention and 1e-2 for the FP32-accumulating baseline at Llama-2-7B
shape) without defining it.  Elementwise |dO|/|O| is unbounded near zero, so
this module reports the normwise forms: max|dO| / max|O_ref| per tensor and
the largest row-wise ||dO_i||_2 / ||O_ref,i||_2.

Tie bias (page 2, "Mechanism 2": the bias is a directional rounding error
triggered by a repeated row maximum; and "More important lessons": errors
under discrete events such as repeated maxima are not zero-mean noise).  A
row whose maximum is attained twice has O close to the midpoint (v_a + v_b)/2
of the tied value rows; the BF16 output rounding there tends to move with the
small exact correction O - H (H = mean of the tied value rows).  The aligned
signed error mean((O - O_ref) * sign(O_ref - H)) measures that directional
bias; the plain signed mean is reported beside it.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def output_errors(o, o_ref) -> Dict[str, float]:
    o, o_ref = _f64(o), _f64(o_ref)
    diff = o - o_ref
    ad = np.abs(diff)
    row_err = np.sqrt((diff ** 2).sum(axis=-1))
    row_ref = np.sqrt((o_ref ** 2).sum(axis=-1))
    with np.errstate(divide="ignore", invalid="ignore"):
        row_rel = np.where(row_ref > 0, row_err / row_ref, np.where(row_err > 0, np.inf, 0.0))
    return {
        "max_abs": float(ad.max()) if ad.size else 0.0,
        "mean_abs": float(ad.mean()) if ad.size else 0.0,
        "max_rel_normwise": float(ad.max() / max(np.abs(o_ref).max(), 1e-300)) if ad.size else 0.0,
        "max_rel_rowwise": float(row_rel.max()) if row_rel.size else 0.0,
        "finite": bool(np.isfinite(o).all()),
    }


def relative_fro(x, ref) -> float:
    """||x - ref||_F / ||ref||_F."""
    x, ref = _f64(x), _f64(ref)
    den = math.sqrt(float((ref ** 2).sum()))
    num = math.sqrt(float(((x - ref) ** 2).sum()))
    return num / den if den > 0 else (0.0 if num == 0 else math.inf)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits): 2^(floor(log2|x|) - 7)."""
    ax = np.abs(_f64(x))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def f16_ulp(x) -> np.ndarray:
    """Spacing of binary16 numbers at |x| (11 significant bits): 2^(floor(log2|x|) - 10),
    and 2^-24 in the subnormal range below 2^-14."""
    ax = np.abs(_f64(x))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -14.0)
    return np.exp2(e - 10.0)


def ulp(x, fmt: str = "bf16") -> np.ndarray:
    return f16_ulp(x) if fmt == "f16" else bf16_ulp(x)


def _mean_se(x: np.ndarray):
    x = x.ravel()
    if x.size == 0:
        return 0.0, 0.0, 0
    m = float(x.mean())
    se = float(x.std(ddof=1) / math.sqrt(x.size)) if x.size > 1 else 0.0
    return m, se, int(x.size)


def tie_bias(o, o_ref, tie_mean, row_mask) -> Dict[str, float]:
    """Signed-error statistics over the rows selected by ``row_mask``.

    o, o_ref, tie_mean: (..., N, d); row_mask: (..., N) bool.
    """
    o, o_ref, hm = _f64(o), _f64(o_ref), _f64(tie_mean)
    diff = o - o_ref
    sel = np.asarray(row_mask, dtype=bool)
    d_rows = diff[sel]
    s_rows = np.sign(o_ref - hm)[sel]
    plain, plain_se, n = _mean_se(d_rows)
    aligned, aligned_se, _ = _mean_se(d_rows * s_rows)
    return {"rows": int(sel.sum()), "elements": n, "plain_mean": plain, "plain_se": plain_se,
            "aligned_mean": aligned, "aligned_se": aligned_se}


def tie_report(o, o_ref, tie_count, tie_mean) -> Dict[str, Dict[str, float]]:
    """tie_bias on rows with a repeated maximum, and on the other rows as control."""
    tied = np.asarray(tie_count) >= 2
    return {"tie_rows": tie_bias(o, o_ref, tie_mean, tied),
            "control_rows": tie_bias(o, o_ref, tie_mean, ~tied)}
