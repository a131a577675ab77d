"""Seeded synthetic inputs for the attention workloads.

This module is shared by the CPU oracle, the GPU parity tests and the
benchmark.  It holds no attention arithmetic: it draws Gaussian tensors,
rounds them to bfloat16 or IEEE binary16 (round-to-nearest-even, the
workload's element type) and, for the tie-heavy
workloads, copies one key row onto another so that a query row sees its
largest score twice.  Picking which key to copy needs the raw dot products
q.k of one head; they are taken in float64 on bf16- or binary16-exact values
(exact, so the order of summation cannot matter) and are used for nothing
else.

Workloads (shapes from the attention layers the pages discuss: GPT-2 small
and medium, Llama-2-7B, and page 1's "critical" N*B = 131072 shape):

  c1  B=1  H=1  N=256  d=64  non-causal, 10% of rows with a repeated max
  c2  B=8  H=12 N=1024 d=64  causal, Q and K times 4, 5% repeated-max rows
  c3  B=64 H=16 N=2048 d=64  causal, K plus a shared rank-4 term (weight 0.5)
  c4  B=4  H=32 N=4096 d=128 causal, plain N(0,1)
  c5  B=16 H=16 N=1024 d=64  causal, 5% repeated-max rows, with dO

and the same c2, c4 and c5 shapes in binary16 (c2h, c4h, c5h: own seeds),
for the FP16 path (page 1 describes the bias and the fix for FP16 and BF16
alike).

Every (b, h) head is drawn from its own counter-seeded PCG64 stream
``default_rng([seed, b, h])`` so that any subset of heads can be rebuilt on
the CPU without drawing the whole tensor; the full tensors handed to the GPU
are the concatenation of the same per-head draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    qk_mult: float = 1.0          # Q and K are multiplied by this before rounding
    tie_frac: float = 0.0         # target fraction of rows with a repeated max
    lowrank_rank: int = 0         # rank of the shared component added to K
    lowrank_weight: float = 0.0
    with_do: bool = False         # also draw dO (backward workloads)
    dtype: str = "bf16"           # element type of the tensors: "bf16" or "f16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def heads(self) -> int:
        return self.B * self.H

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", 1, 1, 256, 64, False, 1001, tie_frac=0.10),
    "c2": Workload("c2", 8, 12, 1024, 64, True, 1002, qk_mult=4.0, tie_frac=0.05),
    "c3": Workload("c3", 64, 16, 2048, 64, True, 1003, lowrank_rank=4, lowrank_weight=0.5),
    "c4": Workload("c4", 4, 32, 4096, 128, True, 1004),
    "c5": Workload("c5", 16, 16, 1024, 64, True, 1005, tie_frac=0.05, with_do=True),
    "c2h": Workload("c2h", 8, 12, 1024, 64, True, 1012, qk_mult=4.0, tie_frac=0.05, dtype="f16"),
    "c4h": Workload("c4h", 4, 32, 4096, 128, True, 1014, dtype="f16"),
    "c5h": Workload("c5h", 16, 16, 1024, 64, True, 1015, tie_frac=0.05, with_do=True, dtype="f16"),
}


# ----------------------------------------------------------------------------
# bf16 encoding of the drawn values (input quantisation only)
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    The generated values are finite, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round to nearest even
    (numpy's float16 conversion)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of binary16 bit patterns to float32."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> 16-bit patterns of the element type."""
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f16":
        return to_f16_bits(x)
    raise ValueError(f"unknown element type {dtype!r}")


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns of the element type -> float32 (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    if dtype == "f16":
        return f16_bits_to_f32(bits)
    raise ValueError(f"unknown element type {dtype!r}")


# ----------------------------------------------------------------------------
# repeated-maximum construction
# ----------------------------------------------------------------------------

def _visible(N: int, causal: bool, i: int) -> int:
    """Number of keys query i can see (keys 0..n-1)."""
    return i + 1 if causal else N


def _make_ties(q: np.ndarray, k_bits: np.ndarray, causal: bool, target: int,
               rng: np.random.Generator, dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """Copy key rows so that at least `target` query rows have a repeated max.

    q: (N, d) float64 (values exact in the element type); k_bits: (N, d)
    uint16 patterns of that type, edited in place on a copy.  Returns (new k_bits, sorted array of every row whose maximum
    is attained at least twice at the end).  Copying K[a] ties every row whose
    argmax is a and that can see b, so the count includes such collateral rows
    and can exceed `target`.

    Procedure: walk the candidate rows in a seeded random order (causal: rows
    i >= 1, since row 0 sees one key).  For row i take a = its visible argmax
    and a partner b drawn uniformly among its visible keys that are neither a
    nor protected; protected keys are every key that currently attains some
    row's maximum, plus all earlier sources and targets.  Set K[b] = K[a].
    Because b attained no row's maximum, removing its old column cannot lower
    any row maximum, so the maxima are updated incrementally from the new
    column alone.
    """
    N, d = q.shape
    k_bits = k_bits.copy()
    kf = decode(k_bits, dtype).astype(np.float64)
    s = q @ kf.T                                   # exact: 16-bit products summed in fp64
    if causal:
        s[np.triu_indices(N, 1)] = -np.inf
    rowmax = s.max(axis=1)
    argsets: List[set] = [set(np.flatnonzero(s[i] == rowmax[i]).tolist()) for i in range(N)]
    protected = set()
    for st in argsets:
        protected |= st
    targeted: List[int] = []
    ntied = sum(1 for st in argsets if len(st) >= 2)

    cand = np.arange(1 if causal else 0, N)
    rng.shuffle(cand)
    for i in cand:
        if ntied >= target:
            break
        i = int(i)
        if len(argsets[i]) >= 2:
            continue
        a = min(argsets[i])
        nvis = _visible(N, causal, i)
        free = np.ones(nvis, dtype=bool)
        free[a] = False
        prot = np.fromiter((j for j in protected if j < nvis), dtype=np.int64)
        free[prot] = False
        pool = np.flatnonzero(free)
        if pool.size == 0:
            continue
        b = int(pool[int(rng.integers(pool.size))])
        k_bits[b] = k_bits[a]
        kf[b] = kf[a]
        col = q @ kf[b]
        if causal:
            col[:b] = -np.inf                      # rows r < b cannot see key b
        for r in np.flatnonzero(col > rowmax):
            before = len(argsets[r]) >= 2
            rowmax[r] = col[r]
            protected.update(argsets[r])
            argsets[r] = {b}
            ntied -= int(before)
        for r in np.flatnonzero(col == rowmax):
            if b not in argsets[r]:
                argsets[r].add(b)
                ntied += int(len(argsets[r]) == 2)
        protected.update((a, b))
        targeted.append(i)
    tie_rows = np.array([r for r in range(N) if len(argsets[r]) >= 2], dtype=np.int64)
    return k_bits, tie_rows


# ----------------------------------------------------------------------------
# per-head and full-tensor generation
# ----------------------------------------------------------------------------

def _lowrank_factors(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    rng = np.random.default_rng([w.seed, 0x10F])
    a = rng.standard_normal((w.N, w.lowrank_rank))
    b = rng.standard_normal((w.d, w.lowrank_rank))
    return a, b


def head(w: Workload, b: int, h: int, lowrank: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """Inputs of one (b, h) head as 16-bit patterns of the workload's element
    type, shape (N, d) each.

    Keys: 'q', 'k', 'v' (and 'do' when the workload has a backward), plus
    'tie_rows' (rows whose maximum raw score repeats after the construction).
    """
    rng = np.random.default_rng([w.seed, b, h])
    shape = (w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32) if w.with_do else None
    if w.qk_mult != 1.0:
        q = q * np.float32(w.qk_mult)
        k = k * np.float32(w.qk_mult)
    if w.lowrank_rank:
        fa, fb = lowrank if lowrank is not None else _lowrank_factors(w)
        k = (k.astype(np.float64) + w.lowrank_weight * (fa @ fb.T) / math.sqrt(w.lowrank_rank)).astype(np.float32)
    out = {"q": encode(q, w.dtype), "k": encode(k, w.dtype), "v": encode(v, w.dtype)}
    if do is not None:
        out["do"] = encode(do, w.dtype)
    tie_rows = np.zeros(0, dtype=np.int64)
    if w.tie_frac > 0:
        target = int(round(w.tie_frac * w.N))
        qf = decode(out["q"], w.dtype).astype(np.float64)
        trng = np.random.default_rng([w.seed, b, h, 0x71E])
        out["k"], tie_rows = _make_ties(qf, out["k"], w.causal, target, trng, w.dtype)
    out["tie_rows"] = tie_rows
    return out


def heads(w: Workload, pairs: Iterable[Tuple[int, int]]) -> List[Dict[str, np.ndarray]]:
    lr = _lowrank_factors(w) if w.lowrank_rank else None
    return [head(w, b, h, lr) for (b, h) in pairs]


def full(w: Workload) -> Dict[str, np.ndarray]:
    """Whole (B, H, N, d) tensors (uint16 patterns of the element type) plus
    tie rows per head."""
    names = ["q", "k", "v"] + (["do"] if w.with_do else [])
    out = {n: np.empty((w.B, w.H, w.N, w.d), dtype=np.uint16) for n in names}
    ties = {}
    lr = _lowrank_factors(w) if w.lowrank_rank else None
    for b in range(w.B):
        for h in range(w.H):
            hd = head(w, b, h, lr)
            for n in names:
                out[n][b, h] = hd[n]
            ties[(b, h)] = hd["tie_rows"]
    out["tie_rows"] = ties
    return out


def sample_pairs(w: Workload, count: int, seed: int = 0) -> List[Tuple[int, int]]:
    """A seeded random subset of (b, h) pairs (all pairs if count >= B*H)."""
    allp = [(b, h) for b in range(w.B) for h in range(w.H)]
    if count >= len(allp):
        return allp
    rng = np.random.default_rng([w.seed, 0x5A3, seed])
    idx = np.sort(rng.choice(len(allp), size=count, replace=False))
    return [allp[i] for i in idx]


def random_bf16(shape: Sequence[int], seed: int, mult: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Plain N(0, mult^2) 16-bit patterns (bf16 unless ``dtype`` says "f16")
    for ad-hoc shapes (edge-case tests)."""
    rng = np.random.default_rng([seed, 0xEDCE])
    return encode(rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(mult), dtype)
