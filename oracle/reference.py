"""Oracle A: exact softmax attention in float64 (test infrastructure only).

Definition followed (page 3, "Flash Attention: from academic breakthrough to
industry standard" -- FlashAttention computes exact attention, so the
operation is softmax(scale * Q K^T) V, with a logsumexp per row for the
backward):

  S_ij  = scale * sum_t q_it k_jt        (S_ij = -inf for j > i when causal)
  r_i   = max_j S_ij
  l_i   = sum_j exp(S_ij - r_i)
  P_ij  = exp(S_ij - r_i) / l_i
  O_i   = sum_j P_ij v_j
  LSE_i = r_i + ln l_i

Backward of L = sum(O * dO) (the standard softmax-attention gradients):

  dP_ij = dO_i . v_j
  D_i   = sum_j P_ij dP_ij
  dS_ij = P_ij (dP_ij - D_i)
  dQ_i  = scale * sum_j dS_ij k_j
  dK_j  = scale * sum_i dS_ij q_i
  dV_j  = sum_i P_ij dO_i

Inputs are any float arrays of shape (..., N, d); they are widened to float64
(bf16 and fp32 values widen exactly).  Causal masking is top-left aligned:
query i sees keys 0..i.  Matrix products use numpy's matmul (a library
primitive); nothing is blocked or reordered beyond the definition.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale: float, causal: bool) -> np.ndarray:
    """S = scale * Q K^T with -inf above the diagonal when causal."""
    q, k = _f64(q), _f64(k)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        n_q, n_k = s.shape[-2], s.shape[-1]
        mask = np.triu(np.ones((n_q, n_k), dtype=bool), 1)
        s = np.where(mask, -np.inf, s)
    return s


def probabilities(q, k, scale: float, causal: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Row-softmax P of the scores, and LSE = r + ln l."""
    s = scores(q, k, scale, causal)
    r = s.max(axis=-1, keepdims=True)
    e = np.exp(s - r)
    l = e.sum(axis=-1, keepdims=True)
    p = e / l
    lse = (r + np.log(l))[..., 0]
    return p, lse


def forward(q, k, v, scale: float, causal: bool) -> Tuple[np.ndarray, np.ndarray]:
    """(O, LSE) in float64."""
    p, lse = probabilities(q, k, scale, causal)
    o = p @ _f64(v)
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV) in float64 for L = sum(O * dO)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _ = probabilities(q, k, scale, causal)
    dp = do @ np.swapaxes(v, -1, -2)
    dvec = (p * dp).sum(axis=-1, keepdims=True)
    ds = p * (dp - dvec)
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    dv = np.swapaxes(p, -1, -2) @ do
    return dq, dk, dv


def tie_metadata(q, k, v, scale: float, causal: bool) -> Dict[str, np.ndarray]:
    """Per row: how many keys attain the exact row maximum, and the mean of
    their value rows.

    Equality is exact float64 equality of the scores.  Bit-identical key rows
    give bit-identical scores because bf16 products summed in float64 are
    exact at these sizes.  Returns {'count': (..., N) int, 'tie_mean': (..., N, d)}.
    """
    s = scores(q, k, scale, causal)
    r = s.max(axis=-1, keepdims=True)
    at_max = (s == r) & np.isfinite(s)
    count = at_max.sum(axis=-1)
    tie_mean = (at_max.astype(np.float64) @ _f64(v)) / np.maximum(count, 1)[..., None]
    return {"count": count, "tie_mean": tie_mean}
