"""Oracle C: the unfused baseline attention with FP32 accumulation, emulated
with its rounding sites (test infrastructure only).

Page 3 ("What did Meta's study find") measures FlashAttention against a
baseline attention that accumulates in FP32, in an isolated BF16 forward
pass: the baseline's maximum relative error at Llama-2-7B shape is given as
about 1e-2 and FlashAttention's as about 1e-1.  The page attributes the gap to
the tiled algorithm rescaling and updating every block on its own.  It does
not spell out the baseline's arithmetic; the reading taken here is the plain
unfused attention with every accumulation in FP32 and the two products on
BF16 operands:

  t_ij  = fl32(q_i . k_j)                      raw dot product, FP32 accumulation
  S_ij  = fl32(t_ij * fl32(scale))             the score matrix, materialised in FP32
                                               (-inf for j > i when causal)
  r_i   = max_j S_ij                           one maximum over the whole row
  e_ij  = fl32(2^fl32(fl32(S_ij - r_i) * fl32(log2 e)))
  l_i   = fl32(sum_j e_ij)                     FP32 (summation order left open)
  P_ij  = bf16(fl32(e_ij * fl32(1 / l_i)))     normalised, then cast to BF16
  O_i   = bf16(fl32(sum_j P_ij v_j))           FP32 accumulation, BF16 output
  LSE_i = fl32(r_i + fl32(fl32(log2 l_i) * fl32(ln 2)))

It differs from FlashAttention (``emulation.forward``) in where the BF16
rounding of the probabilities sits: here the probabilities are normalised
before the cast (so a row's BF16 probabilities need not sum to 1), there the
unnormalised ones in [0, 1] are cast and the output is divided by the FP32
sum at the end.

Sums whose order the kernel leaves to the hardware (the dot products, l, the
PV accumulation) are taken here in float64 and rounded once; the GPU's FP32
accumulation differs from that by a few FP32 ulps, far below the BF16 sites.
``no_round=True`` removes every rounding and must then equal the exact oracle
(``reference.forward``) to ~1e-12.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .emulation import LN2, LOG2E, bf16, fl32


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale: float, causal: bool, *, no_round: bool = False) -> np.ndarray:
    """The FP32 score matrix S of the baseline (-inf above the diagonal when causal)."""
    r32 = _ident if no_round else fl32
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    sc = scale if no_round else float(np.float32(scale))
    t = r32(q @ np.swapaxes(k, -1, -2))
    s = r32(t * sc)
    if causal:
        n_q, n_k = s.shape[-2], s.shape[-1]
        s = np.where(np.triu(np.ones((n_q, n_k), dtype=bool), 1), -np.inf, s)
    return s


def softmax(s, *, no_round: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax of an FP32 score matrix: (P rounded to BF16, LSE)."""
    r32, rb16 = (_ident, _ident) if no_round else (fl32, bf16)
    l2e = LOG2E if no_round else float(np.float32(LOG2E))
    ln2 = LN2 if no_round else float(np.float32(LN2))
    r = s.max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = r32(np.exp2(r32(r32(s - r) * l2e)))       # masked entries: exp2(-inf) = 0
    l = r32(e.sum(axis=-1, keepdims=True))
    inv = r32(1.0 / l)
    p = rb16(r32(e * inv))
    lse = r32(r[..., 0] + r32(r32(np.log2(l[..., 0])) * ln2))
    return p, lse


def forward(q, k, v, scale: float, causal: bool, *, no_round: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(O, LSE) of the baseline for (..., N, d) inputs (values exact in bf16)."""
    r32, rb16 = (_ident, _ident) if no_round else (fl32, bf16)
    s = scores(q, k, scale, causal, no_round=no_round)
    p, lse = softmax(s, no_round=no_round)
    o = rb16(r32(p @ np.asarray(v, dtype=np.float64)))
    return o, lse
