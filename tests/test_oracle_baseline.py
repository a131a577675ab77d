"""Pins for the unfused FP32-accumulating baseline emulation (oracle.baseline).

* With every rounding switched off it must reproduce the exact oracle: the
  baseline is plain softmax attention, computed in one piece (page 3, "What did
  Meta's study find").
* A hand-derived worked example (tests/golden/baseline_three_way_tie.json)
  pins its rounding sites: the probabilities are normalised before their BF16
  cast (three tied keys get bf16(1/3) each, which sum to more than 1) and the
  output is rounded once at the end.  The same example pins FlashAttention's
  different site (unnormalised probabilities of exactly 1, division at the
  end) through the blocked emulation.
* Closed forms: a single dominant key returns its value row exactly; a
  power-of-two number of identical keys gives probabilities 1/n exactly and so
  the correctly rounded mean; causal row 0 is v_0.
* On unit-variance inputs its error against the exact oracle sits inside the
  forward's gates.
"""
import json
import math
import os

import numpy as np
import pytest

import fa_inputs as F
from oracle import baseline as C
from oracle import emulation as B
from oracle import metrics as Mt
from oracle import reference as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, mult=1.0):
    return F.decode(F.random_bf16(shape, seed, mult), "bf16").astype(np.float64)


@pytest.mark.parametrize("N,d,causal", [(1, 64, False), (7, 16, True), (33, 64, False), (70, 128, True)])
def test_no_round_equals_exact_oracle(N, d, causal):
    q, k, v = (_rand((2, N, d), 40 + i, 2.0 if i < 2 else 1.0) for i in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = C.forward(q, k, v, scale, causal, no_round=True)
    o_ref, lse_ref = A.forward(q, k, v, scale, causal)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12
    p, _ = C.softmax(C.scores(q, k, scale, causal, no_round=True), no_round=True)
    p_ref, _ = A.probabilities(q, k, scale, causal)
    assert np.max(np.abs(p - p_ref)) < 1e-14


def test_golden_three_way_tie():
    with open(os.path.join(GOLDEN, "baseline_three_way_tie.json")) as f:
        g = json.load(f)
    q, k, v = (np.array(g[n], dtype=np.float64)[None] for n in ("q", "k", "v"))
    o, lse = C.forward(q, k, v, g["scale"], False)
    assert o[0, 0].tolist() == g["o_baseline"]
    assert abs(lse[0, 0] - g["lse"]) < 1e-6
    p, _ = C.softmax(C.scores(q, k, g["scale"], False))
    assert np.all(p == g["p_baseline_bf16"])
    for stab in (False, True):
        o_fa, lse_fa = B.forward(q, k, v, g["scale"], False, stabilize=stab)
        assert o_fa[0, 0].tolist() == g["o_flash"]
        assert abs(lse_fa[0, 0] - g["lse"]) < 1e-6
    o_ex, _ = A.forward(q, k, v, g["scale"], False)
    assert np.allclose(o_ex[0, 0], g["o_exact"], rtol=0, atol=1e-15)


def test_dominant_key_returns_its_value_row():
    d, N = 64, 40
    q = np.zeros((1, N, d))
    k = np.zeros((1, N, d))
    q[..., 0] = 1.0
    k[0, 13, 0] = 64.0        # raw score 64 for key 13, 0 for every other key
    scale = 8.0               # scaled: 512 against 0
    v = _rand((1, N, d), 7)
    o, lse = C.forward(q, k, v, scale, False)
    assert np.array_equal(o[0], np.broadcast_to(v[0, 13], (N, d)))
    assert np.allclose(lse, 512.0, rtol=0, atol=1e-4)


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_power_of_two_identical_keys_give_the_rounded_mean(n):
    d = 64
    q = _rand((1, 3, d), 11)
    k = np.broadcast_to(_rand((1, 1, d), 12), (1, n, d)).copy()
    v = _rand((1, n, d), 13)
    o, lse = C.forward(q, k, v, 1.0 / 8.0, False)
    p, _ = C.softmax(C.scores(q, k, 1.0 / 8.0, False))
    assert np.all(p == 1.0 / n)
    assert np.array_equal(o[0], np.broadcast_to(B.bf16(v[0].mean(axis=0)), (3, d)))


def test_causal_row_zero_is_the_first_value_row():
    q, k, v = (_rand((3, 50, 64), 20 + i) for i in range(3))
    o, _ = C.forward(q, k, v, 0.125, True)
    assert np.array_equal(o[:, 0], v[:, 0])


def test_error_inside_the_forward_gates_on_unit_variance_inputs():
    q, k, v = (_rand((4, 256, 64), 30 + i) for i in range(3))
    scale = 0.125
    for causal in (False, True):
        o, lse = C.forward(q, k, v, scale, causal)
        o_ref, lse_ref = A.forward(q, k, v, scale, causal)
        e = Mt.output_errors(o, o_ref)
        assert e["max_abs"] <= 1.5e-2 and e["mean_abs"] <= 2e-3
        assert np.max(np.abs(lse - lse_ref)) < 1e-5
