"""Seeded random shapes through every entry point, against the exact oracle.

Twenty-four (B, H, N, d, causal, range count) cases drawn once from a fixed
seed (N from 1 to 700, d 64 or 128, a few heads): the forward, the backward,
the split-key forward (with a random range count) and the baseline each meet
their gates, and the forward with the fix on and off agree bitwise on every
row the fix never touched.  The shapes fall on and off every tile boundary
(64-key blocks, 128-row query blocks, 32-row waves).
"""
import numpy as np
import pytest

from oracle import metrics as Mt
from oracle import reference as REF

from gpu_util import head_f64, random_case, say, to_f64, LSE_TOL, lse_err

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261203)
CASES = [(int(_rng.integers(1, 3)), int(_rng.integers(1, 4)), int(_rng.integers(1, 701)),
          int(_rng.choice([64, 128])), bool(_rng.integers(0, 2)), int(_rng.integers(2, 9)), 500 + i)
         for i in range(24)]


@pytest.fixture(scope="module")
def fa():
    import torch
    import precision_numerics_fa_amd as fa
    assert torch.cuda.is_available()
    fa.load()
    return fa


@pytest.mark.parametrize("B,H,N,d,causal,splits,seed", CASES)
def test_random_shape_every_entry_point(fa, B, H, N, d, causal, splits, seed):
    say(f"random shape B={B} H={H} N={N} d={d} causal={causal} splits={splits} seed={seed}")
    bits, dev = random_case(B, H, N, d, seed=seed, with_do=True)
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (head_f64(bits[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = REF.forward(q, k, v, scale, causal)
    g_ref = REF.backward(q, k, v, do, scale, causal)

    def gate(o, lse, what):
        e = Mt.output_errors(to_f64(o), o_ref)
        assert e["max_abs"] <= 1.5e-2 and e["mean_abs"] <= 2e-3 and e["finite"], (what, e)
        assert lse_err(to_f64(lse), lse_ref) <= LSE_TOL, what

    o_on, lse_on, flags = fa.fwd_diag(dev["q"], dev["k"], dev["v"], causal=causal, stabilize=True)
    gate(o_on, lse_on, "fwd fix on")
    o_off, lse_off = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, stabilize=False)
    gate(o_off, lse_off, "fwd fix off")
    untouched = to_f64(flags) == 0
    assert np.array_equal(to_f64(o_on)[untouched], to_f64(o_off)[untouched])

    dq, dk, dv = fa.bwd(dev["q"], dev["k"], dev["v"], o_on, dev["do"], lse_on, causal=causal)
    for name, g, r in (("dq", dq, g_ref[0]), ("dk", dk, g_ref[1]), ("dv", dv, g_ref[2])):
        assert Mt.relative_fro(to_f64(g), r) <= 5e-2, name

    o_s, lse_s = fa.fwd_split(dev["q"], dev["k"], dev["v"], splits, causal=causal, stabilize=True)
    gate(o_s, lse_s, "split")
    o_b, lse_b = fa.base_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    gate(o_b, lse_b, "baseline")
