"""Pins for the error statistics (oracle.metrics) on hand-computed cases.

Each expected value below is worked out by hand in the comment beside it, so
that a plausible slip in a statistic (a missing square root, a swapped sign,
a mean over the wrong rows, the wrong ulp exponent) fails here rather than
silently loosening or tightening every gate that uses it.
"""
import math

import numpy as np
import pytest

from oracle import metrics as Mt


def test_output_errors_hand_case():
    o = np.array([[1.0, 2.0], [3.0, 4.0]])
    o_ref = np.array([[1.0, 2.5], [3.0, 3.0]])
    # diff = [[0, -0.5], [0, 1]]: max |diff| = 1, mean = 1.5 / 4 = 0.375;
    # max |O_ref| = 3, so max_rel_normwise = 1/3;
    # row 0: ||diff|| = 0.5, ||ref|| = sqrt(1 + 6.25) = sqrt(7.25) -> 0.1857;
    # row 1: ||diff|| = 1, ||ref|| = sqrt(18) -> 0.2357 = max_rel_rowwise
    e = Mt.output_errors(o, o_ref)
    assert e["max_abs"] == 1.0
    assert e["mean_abs"] == 0.375
    assert e["max_rel_normwise"] == pytest.approx(1.0 / 3.0, rel=1e-15)
    assert e["max_rel_rowwise"] == pytest.approx(1.0 / math.sqrt(18.0), rel=1e-15)
    assert e["finite"] is True
    # a zero reference row with a non-zero error is an infinite row ratio;
    # a zero row with no error is 0; a NaN output is reported as not finite
    z = Mt.output_errors(np.array([[0.0, 1.0], [0.0, 0.0]]), np.zeros((2, 2)))
    assert z["max_rel_rowwise"] == math.inf
    assert Mt.output_errors(np.zeros((1, 2)), np.zeros((1, 2)))["max_rel_rowwise"] == 0.0
    assert Mt.output_errors(np.array([[np.nan, 0.0]]), np.zeros((1, 2)))["finite"] is False


def test_relative_fro_hand_case():
    # x - ref = [3, 4] (norm 5), ref = [6, 8] (norm 10): 5 / 10 = 0.5
    # (without the square roots it would read 25 / 100 = 0.25)
    ref = np.array([6.0, 8.0])
    assert Mt.relative_fro(ref + np.array([3.0, 4.0]), ref) == 0.5
    # Frobenius over every axis: a (2, 2) error [[1, 1], [1, 1]] against a
    # reference of norm 4 ([[2, 2], [2, 2]]) is 2 / 4
    assert Mt.relative_fro(np.full((2, 2), 3.0), np.full((2, 2), 2.0)) == 0.5
    assert Mt.relative_fro(np.zeros(3), np.zeros(3)) == 0.0
    assert Mt.relative_fro(np.ones(3), np.zeros(3)) == math.inf


def test_tie_bias_sign_convention_hand_case():
    # Row 0 is selected: O_ref = [1.25, 2], H = [1, 3], so sign(O_ref - H) =
    # [+1, -1].  O = [1.5, 1.5]: diff = [0.25, -0.5].
    #   plain   = mean(0.25, -0.5) = -0.125; sample sd = 0.75/sqrt(2), se = 0.375
    #   aligned = mean(0.25 * 1, -0.5 * -1) = 0.375; sd = 0.25/sqrt(2), se = 0.125
    # An error that moves O away from H (towards the side the exact correction
    # lies on) counts positive.  Row 1 is not selected and must not count.
    o = np.array([[1.5, 1.5], [100.0, -100.0]])
    o_ref = np.array([[1.25, 2.0], [0.0, 0.0]])
    hm = np.array([[1.0, 3.0], [0.0, 0.0]])
    r = Mt.tie_bias(o, o_ref, hm, np.array([True, False]))
    assert r["rows"] == 1 and r["elements"] == 2
    assert r["plain_mean"] == -0.125 and r["plain_se"] == pytest.approx(0.375, rel=1e-15)
    assert r["aligned_mean"] == 0.375 and r["aligned_se"] == pytest.approx(0.125, rel=1e-15)
    # tie_report splits on the count: >= 2 is a tie row, the rest the control
    rep = Mt.tie_report(o, o_ref, np.array([2, 1]), hm)
    assert rep["tie_rows"]["aligned_mean"] == 0.375
    assert rep["control_rows"]["rows"] == 1
    # row 1: diff = [100, -100], sign(O_ref - H) = [0, 0] -> aligned 0, plain 0
    assert rep["control_rows"]["plain_mean"] == 0.0 and rep["control_rows"]["aligned_mean"] == 0.0
    # no selected rows: zeros, not NaN
    empty = Mt.tie_bias(o, o_ref, hm, np.array([False, False]))
    assert empty["elements"] == 0 and empty["aligned_mean"] == 0.0


def test_ulp_spacings_hand_values():
    # bf16 keeps 8 significant bits: spacing 2^(e - 7) for |x| in [2^e, 2^(e+1))
    assert Mt.bf16_ulp(1.0) == 2.0 ** -7 and Mt.bf16_ulp(1.99) == 2.0 ** -7
    assert Mt.bf16_ulp(0.75) == 2.0 ** -8 and Mt.bf16_ulp(-4.5) == 2.0 ** -5
    # binary16: 11 significant bits, subnormal spacing 2^-24 below 2^-14
    assert Mt.f16_ulp(1.0) == 2.0 ** -10 and Mt.f16_ulp(3.0) == 2.0 ** -9
    assert Mt.f16_ulp(2.0 ** -20) == 2.0 ** -24 and Mt.f16_ulp(2.0 ** -14) == 2.0 ** -24
    assert Mt.ulp(1.0, "f16") == 2.0 ** -10 and Mt.ulp(1.0) == 2.0 ** -7
