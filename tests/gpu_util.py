"""Helpers for the GPU parity tests: host<->device transfer of bf16 bit
patterns and oracle comparisons on selected heads."""
import sys

import numpy as np

import fa_inputs as F


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def head_f64(bits: np.ndarray) -> np.ndarray:
    return F.bf16_bits_to_f32(bits).astype(np.float64)


def device_inputs(w: F.Workload):
    """Full (B,H,N,d) tensors of a workload on the GPU, plus the host bits."""
    full = F.full(w)
    dev = {n: to_dev(full[n]) for n in ("q", "k", "v", "do") if n in full}
    return full, dev


def random_case(B, H, N, d, seed, mult=1.0, with_do=False):
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    bits = {n: F.random_bf16((B, H, N, d), seed * 10 + i, mult) for i, n in enumerate(names)}
    return bits, {n: to_dev(b) for n, b in bits.items()}
