"""Pins for the BF16 blocked emulation (oracle.emulation).

* With every rounding switched off (float64, no casts) the blocked online
  recurrence must reproduce the exact oracle for any block size and for both
  the plain and the stabilised shift: softmax is invariant to the shift, and
  the tiling reorganises an exact computation (page 3, on FlashAttention's
  origins; page 2, on the fix changing only m).
* The running tie count must end equal to a brute-force count of the row
  maximum; the fix must act only on rows whose maximum repeats (page 2,
  "Mechanism 2": detect whether the maximum occurs more than once) and must
  leave the largest probability strictly below 1, in bf16 too.
* The rounding primitives are checked against PyTorch's own float32 ->
  bfloat16 conversion (round to nearest even).
* A hand-derived worked example (tests/golden/tie_midpoint.json) pins the
  rounding sites: the bf16 cast of P before the PV product, the unrounded row
  sum and the bf16 output cast; tie_midpoint_f16.json pins the same sites in
  binary16.
* The binary16 rounding is checked against PyTorch's float32 -> float16
  conversion and hand-computed ties, subnormals and overflow, and the
  binary16 emulation must be closer to the exact result than the bf16 one on
  the same (bf16-exact) inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import fa_inputs as F
from oracle import emulation as B
from oracle import metrics as Mt
from oracle import reference as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _head(name, b=0, h=0, **kw):
    w = F.WORKLOADS[name].with_shape(**kw) if kw else F.WORKLOADS[name]
    hd = F.head(w, b, h)
    return w, [F.decode(hd[n], w.dtype).astype(np.float64) for n in ("q", "k", "v")], hd


# ---------------------------------------------------------------- primitives

def test_bf16_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -1.00390625, 3.0e38, 3.4e38, -3.4e38,
         np.inf, -np.inf, 1e-40, -1e-42, 0.1353352814912796],
    ]).astype(np.float32)
    mine = B.bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)
    assert np.isnan(B.bf16(np.array([np.nan]))).all()


def test_f16_matches_torch_and_hand_values():
    rng = np.random.default_rng(6)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        [0.0, -0.0, 1.0, 65504.0, 70000.0, -70000.0, 1e-8, -3e-8, 0.1353352814912796],
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(B.f16(x), ref)
    hand = {
        1.0 + 2.0 ** -11: 1.0,                       # tie: to the even neighbour 1.0
        1.0 + 3 * 2.0 ** -11: 1.0 + 2.0 ** -9,       # tie: to the even neighbour above
        1.0 + 2.0 ** -11 + 2.0 ** -20: 1.0 + 2.0 ** -10,
        65519.0: 65504.0,                            # below the overflow midpoint
        65520.0: np.inf,                             # the midpoint rounds to inf
        2.0 ** -25: 0.0,                             # half the smallest subnormal: to even (0)
        3 * 2.0 ** -26: 2.0 ** -24,
        2.0 ** -14 + 2.0 ** -25: 2.0 ** -14,         # subnormal-range spacing is 2^-24
    }
    for a, b in hand.items():
        assert B.f16(np.array([a]))[0] == b, (a, b)
    assert np.isnan(B.f16(np.array([np.nan]))).all()


def test_ulp_helpers():
    assert Mt.f16_ulp(np.array([1.0, 1.5, 0.5, 2.0 ** -20, 65504.0])).tolist() == \
        [2.0 ** -10, 2.0 ** -10, 2.0 ** -11, 2.0 ** -24, 32.0]
    assert Mt.bf16_ulp(np.array([1.0, 3.0])).tolist() == [2.0 ** -7, 2.0 ** -6]


def test_fl32_is_float32_rounding():
    # hand-derived: 1 + 2^-30 is below half an ulp of 1; 1/3 rounds to
    # 11184811 * 2^-25; 1e-45 to the smallest subnormal 2^-149; 3.5e38 lies
    # past the largest finite float32 plus half its ulp, so it overflows
    x = np.array([1.0 + 2.0 ** -30, 1.0 / 3.0, 1e-45, 3.5e38, -(1.0 + 3 * 2.0 ** -24)])
    want = [1.0, 11184811 * 2.0 ** -25, 2.0 ** -149, np.inf, -(1.0 + 2.0 ** -22)]
    assert B.fl32(x).tolist() == want


# ---------------------------------------------------------------- shift rule

def test_shift_rule_values():
    R = np.array([3.25, 64.0, -5.5, -64.0, 0.0, 1e-3, 72.13475036621094, 200.5, -100.25])
    tied = np.ones_like(R, dtype=bool)
    M = B.shift_rule(R, tied, True, B.DELTA_MIN, B.DELTA_MAX, no_round=True)
    expect = np.array([6.5, 128.0, 0.0, 0.0, 1.0 / 16, 1e-3 + 1.0 / 16,
                       72.13475036621094 + 40.13475036621094,
                       200.5 + 40.5,                       # 200.5 folded by 5*32
                       -100.25 + 36.25])                   # 100.25 folded by 2*32
    assert np.allclose(M, expect, rtol=0, atol=1e-12)
    # no tie, or fix off: no shift
    assert np.array_equal(B.shift_rule(R, ~tied, True, B.DELTA_MIN, B.DELTA_MAX, True), R)
    assert np.array_equal(B.shift_rule(R, tied, False, B.DELTA_MIN, B.DELTA_MAX, True), R)
    # the fold keeps the fractional part and lands in (delta_max - 32, delta_max]
    big = np.linspace(64.01, 5000.0, 777)
    d = B.shift_rule(big, np.ones_like(big, bool), True, B.DELTA_MIN, B.DELTA_MAX, True) - big
    assert ((d > 32.0) & (d <= 64.0)).all()
    k = (big - d) / 32.0
    assert np.array_equal(k, np.round(k))


# ---------------------------------------------------------------- no-round equality

@pytest.mark.parametrize("stabilize", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 16, 64, 128, 256])
def test_no_round_equals_exact_oracle(block, causal, stabilize):
    w, (q, k, v), _ = _head("c1", causal=causal, N=200)
    o, lse = A.forward(q, k, v, w.scale, causal)
    ob, lb = B.forward(q, k, v, w.scale, causal, block=block, stabilize=stabilize, no_round=True)
    assert np.abs(ob - o).max() <= 1e-12
    assert np.abs(lb - lse).max() <= 1e-12


def test_no_round_backward_equals_exact_oracle():
    w, (q, k, v), _ = _head("c5", N=96)
    do = np.random.default_rng(3).standard_normal(q.shape)
    o, lse = A.forward(q, k, v, w.scale, True)
    dq, dk, dv = A.backward(q, k, v, do, w.scale, True)
    eq, ek, ev = B.backward(q, k, v, o, do, lse, w.scale, True, no_round=True)
    for a, b in ((eq, dq), (ek, dk), (ev, dv)):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


# ---------------------------------------------------------------- tie bookkeeping

@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_running_count_equals_brute_force_count(name):
    w, (q, k, v), hd = _head(name, N=256) if name != "c1" else _head(name)
    for block in (16, 64, 128):
        _, _, st = B.forward(q, k, v, w.scale, w.causal, block=block, stabilize=True, return_state=True)
        # brute force on the same fp32 raw scores the emulation uses
        t = B.fl32(q @ k.T)
        if w.causal:
            t = np.where(np.triu(np.ones(t.shape, bool), 1), -np.inf, t)
        brute = (t == t.max(axis=1, keepdims=True)).sum(axis=1)
        assert np.array_equal(st["count"], brute)
        # exact fp64 ties (oracle A) are a subset of the fp32 ties
        exact = A.tie_metadata(q, k, v, w.scale, w.causal)["count"]
        assert ((exact >= 2) <= (brute >= 2)).all()
        assert set(np.flatnonzero(exact >= 2)) == set(hd["tie_rows"].tolist())


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_fix_acts_only_on_repeated_max_and_stays_below_one(name, block):
    w, (q, k, v), hd = _head(name, N=512) if name == "c2" else _head(name)
    o0, l0, s0 = B.forward(q, k, v, w.scale, w.causal, block=block, stabilize=False, return_state=True)
    o1, l1, s1 = B.forward(q, k, v, w.scale, w.causal, block=block, stabilize=True, return_state=True)
    never = ~s1["ever_shifted"]
    assert never.sum() > 0 and (~never).sum() >= len(hd["tie_rows"])
    assert np.array_equal(o0[never], o1[never])
    assert np.array_equal(l0[never], l1[never])
    shifted = s1["ever_shifted"]
    assert (s1["pmax_shifted_bf16"][shifted] < 1.0).all()
    assert not s0["ever_shifted"].any()


# ---------------------------------------------------------------- accuracy

@pytest.mark.parametrize("stabilize", [False, True])
def test_rounded_emulation_within_tolerance_c1(stabilize):
    w, (q, k, v), _ = _head("c1")
    o, lse = A.forward(q, k, v, w.scale, w.causal)
    ob, lb = B.forward(q, k, v, w.scale, w.causal, block=64, stabilize=stabilize)
    e = Mt.output_errors(ob, o)
    assert e["max_abs"] <= 1.5e-2 and e["mean_abs"] <= 2e-3
    assert np.abs(lb - lse).max() <= 1e-5


def test_binary16_emulation_is_closer_than_bf16():
    """The binary16 rounding sites have 3 more significant bits than bf16, so on
    the same inputs (bf16 values, exact in binary16 here) the emulated output
    error against the exact oracle shrinks by about 2^3."""
    w, (q, k, v), _ = _head("c1")
    assert np.array_equal(B.f16(q), q) and np.array_equal(B.f16(k), k) and np.array_equal(B.f16(v), v)
    o, _ = A.forward(q, k, v, w.scale, w.causal)
    for stab in (False, True):
        eb = np.abs(B.forward(q, k, v, w.scale, False, block=64, stabilize=stab)[0] - o).mean()
        eh = np.abs(B.forward(q, k, v, w.scale, False, block=64, stabilize=stab, fmt="f16")[0] - o).mean()
        assert eh < eb / 4, (stab, eh, eb)
        assert eh > eb / 32, (stab, eh, eb)


def test_rounded_f16_emulation_within_tolerance():
    w, (q, k, v), hd = _head("c5h", N=256)
    assert w.dtype == "f16"
    do = F.decode(hd["do"], "f16").astype(np.float64)
    o, lse = A.forward(q, k, v, w.scale, True)
    ob, lb = B.forward(q, k, v, w.scale, True, block=64, stabilize=True, fmt="f16")
    e = Mt.output_errors(ob, o)
    assert e["max_abs"] <= 2e-3 and e["mean_abs"] <= 2.5e-4
    dq, dk, dv = A.backward(q, k, v, do, w.scale, True)
    eq, ek, ev = B.backward(q, k, v, ob, do, lb, w.scale, True, fmt="f16")
    for a, b in ((eq, dq), (ek, dk), (ev, dv)):
        assert Mt.relative_fro(a, b) <= 1e-2


def test_rounded_backward_within_tolerance():
    w, (q, k, v), _ = _head("c5", N=256)
    do = F.bf16_bits_to_f32(F.head(F.WORKLOADS["c5"].with_shape(N=256), 0, 0)["do"]).astype(np.float64)
    ob, lb = B.forward(q, k, v, w.scale, True, block=64, stabilize=True)
    dq, dk, dv = A.backward(q, k, v, do, w.scale, True)
    eq, ek, ev = B.backward(q, k, v, ob, do, lb, w.scale, True)
    for a, b in ((eq, dq), (ek, dk), (ev, dv)):
        assert Mt.relative_fro(a, b) <= 5e-2


# ---------------------------------------------------------------- worked example

def test_hand_worked_tie_midpoint():
    g = json.load(open(os.path.join(GOLDEN, "tie_midpoint.json")))
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    o_off, lse_off = B.forward(q, k, v, g["scale"], False, block=64, stabilize=False)
    o_on, lse_on, st = B.forward(q, k, v, g["scale"], False, block=64, stabilize=True, return_state=True)
    o_ex, lse_ex = A.forward(q, k, v, g["scale"], False)
    assert o_ex[0, 0] == g["o_exact"]
    assert o_off[0, 0] == g["o_fix_off"]
    assert o_on[0, 0] == g["o_fix_on"]
    assert st["pmax_shifted_bf16"][0] == g["p_fix_on_bf16"]
    assert abs(lse_off[0] - g["lse"]) <= 1e-6 and abs(lse_on[0] - g["lse"]) <= 1e-6
    # same probabilities when the repeated maximum is negative (shift to 0)
    o_neg = B.forward(-q, k, v, g["scale"], False, block=64, stabilize=True)[0]
    assert o_neg[0, 0] == g["o_fix_on"]
    # one block per key gives the same result: the tie spans two blocks
    o_split = B.forward(q, k, v, g["scale"], False, block=1, stabilize=True)[0]
    assert o_split[0, 0] == g["o_fix_on"]
    # folded shift above delta_max
    fq, fk = np.array(g["fold_q"]), np.array(g["fold_k"])
    _, _, st = B.forward(fq, fk, v, g["scale"], False, block=64, stabilize=True, return_state=True)
    assert st["shift"][0] == np.float32(g["fold_R"] + g["fold_delta"])
    # the shifts, outputs and LSE the GPU check of this example compares against
    for qq, key, lse_key in ((q, "", "lse"), (-q, "neg_", "neg_lse"), (fq, "fold_", "fold_lse")):
        kk = fk if key == "fold_" else k
        for stab, suffix in ((False, "fix_off"), (True, "fix_on")):
            o_s, l_s, st = B.forward(qq, kk, v, g["scale"], False, block=64, stabilize=stab, return_state=True)
            assert st["shift"][0] == g[key + "M_" + suffix]
            if key:
                assert abs(l_s[0] - g[lse_key]) <= 4e-6
            if key == "fold_":
                assert o_s[0, 0] == g["fold_o_" + suffix]


def test_hand_worked_tie_midpoint_f16():
    g = json.load(open(os.path.join(GOLDEN, "tie_midpoint_f16.json")))
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    o_off, lse_off = B.forward(q, k, v, g["scale"], False, block=64, stabilize=False, fmt="f16")
    o_on, lse_on, st = B.forward(q, k, v, g["scale"], False, block=64, stabilize=True, return_state=True,
                                 fmt="f16")
    assert A.forward(q, k, v, g["scale"], False)[0][0, 0] == g["o_exact"]
    assert o_off[0, 0] == g["o_fix_off"]
    assert o_on[0, 0] == g["o_fix_on"]
    assert st["pmax_shifted_bf16"][0] == g["p_fix_on_f16"]
    assert abs(lse_off[0] - g["lse"]) <= 1e-6 and abs(lse_on[0] - g["lse"]) <= 1e-6


def test_binary16_rule_keeps_the_largest_probability_representable():
    """Why binary16 has its own fold.  With the bf16 constants (|R| up to 64)
    the largest probability 2^-|R| of a shifted row underflows in binary16 once
    |R| > 24 and the row's output is lost; folding |R| into (0, 1] keeps it in
    [1/2, 1) and the output within tolerance."""
    w, (q, k, v), _ = _head("c2h", N=512)
    o, _ = A.forward(q, k, v, w.scale, True)
    ob, _, st = B.forward(q, k, v, w.scale, True, stabilize=True, fmt="f16", return_state=True)
    shifted = st["ever_shifted"]
    assert shifted.sum() >= 10
    pm = st["pmax_shifted_bf16"][shifted]
    assert (pm >= 0.5).all() and (pm < 1.0).all()
    assert np.abs(ob - o).max() <= 2e-2
    bad, _, st2 = B.forward(q, k, v, w.scale, True, stabilize=True, fmt="f16", return_state=True,
                            delta_max=B.DELTA_MAX, fold=B.FOLD)
    assert (st2["pmax_shifted_bf16"][shifted] == 0.0).any()
    assert np.abs(bad - o).max() > 0.1


def _bwd_golden():
    g = json.load(open(os.path.join(GOLDEN, "backward_rounding_sites.json")))
    return g, {n: np.array(g[n], dtype=np.float64) for n in ("q", "k", "v", "o", "do", "lse")}


def test_hand_worked_backward_rounding_sites():
    """tests/golden/backward_rounding_sites.json: bf16(P) into dV, bf16(dS)
    into dK and dQ, and D from the bf16 forward output, each visible in the
    result (page 1, section 4.3)."""
    g, a = _bwd_golden()
    dq, dk, dv = B.backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], g["scale"], False)
    assert np.array_equal(dq, np.array(g["dq"]))
    assert np.array_equal(dk, np.array(g["dk"]))
    assert np.array_equal(dv, np.array(g["dv"]))
    # the example's probabilities are the fp32 value it states
    t = a["q"] @ a["k"].T
    assert (t == 0.0).all() and B.fl32(2.0 ** -0.5) == g["p_fp32"]
    # D taken from the exact output (v0 + v1) / 2 instead of the bf16 O: dK_0 is no longer 0
    o_exact = A.forward(a["q"], a["k"], a["v"], g["scale"], False)[0]
    assert o_exact[0, 0] == 1.00390625
    _, dk_x, _ = B.backward(a["q"], a["k"], a["v"], o_exact, a["do"], a["lse"], g["scale"], False)
    assert dk_x[0, 0] != 0.0


@pytest.mark.parametrize("skip, tensor, value", [(1, "dv", "dv_without_p_cast"),
                                                 (3, "dk", "dk1_without_ds_cast"),
                                                 (5, "dq", "dk1_without_ds_cast")])
def test_backward_golden_catches_a_dropped_rounding_site(monkeypatch, skip, tensor, value):
    """Plant each mistake in the oracle: make the n-th 16-bit rounding of the
    backward a no-op (call 1 is bf16(P) for dV, 3 and 5 are bf16(dS) for dK
    and dQ; the even calls round the results) and check that the golden
    example then fails exactly where its derivation says."""
    g, a = _bwd_golden()
    real = B._rounders

    def planted(no_round, fmt="bf16"):
        r32, rb = real(no_round, fmt)
        calls = [0]

        def rb_planted(x):
            calls[0] += 1
            return np.asarray(x, dtype=np.float64) if calls[0] == skip else rb(x)
        return r32, rb_planted

    monkeypatch.setattr(B, "_rounders", planted)
    dq, dk, dv = B.backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], g["scale"], False)
    got = {"dq": dq[0, 1], "dk": dk[1, 0], "dv": dv[0, 0]}[tensor]
    assert got == g[value]
    assert got != {"dq": g["dq"][0][1], "dk": g["dk"][1][0], "dv": g["dv"][0][0]}[tensor]
