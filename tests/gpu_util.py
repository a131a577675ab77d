"""Helpers for the GPU parity tests: host<->device transfer of 16-bit
patterns (bf16 or binary16) and oracle comparisons on selected heads."""
import sys

import numpy as np

import fa_inputs as F


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, dtype: str = "bf16"):
    import torch
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt)
    return t.cuda()


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def head_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    return F.decode(bits, dtype).astype(np.float64)


def device_inputs(w: F.Workload):
    """Full (B,H,N,d) tensors of a workload on the GPU, plus the host bits."""
    full = F.full(w)
    dev = {n: to_dev(full[n], w.dtype) for n in ("q", "k", "v", "do") if n in full}
    return full, dev


def random_case(B, H, N, d, seed, mult=1.0, with_do=False, dtype="bf16"):
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    bits = {n: F.random_bf16((B, H, N, d), seed * 10 + i, mult, dtype) for i, n in enumerate(names)}
    return bits, {n: to_dev(b, dtype) for n, b in bits.items()}


def lse_err(got, ref) -> float:
    """Largest LSE error, absolute where |LSE| <= 1 and relative above (fp32
    LSE of peaked rows is large, and its spacing grows with it)."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max())


# LSE gate: the measured errors are ~1.5e-6 (fp32 log2 / exp2 of the kernels)
LSE_TOL = 1e-5
