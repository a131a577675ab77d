"""Pins for the exact float64 oracle (oracle.reference).

Each test checks the oracle against something other than itself: a closed
form, a scalar brute force with math.fsum, a library routine (PyTorch's
scaled_dot_product_attention and autograd in float64 on the CPU, SciPy's
logsumexp), or central finite differences.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import reference as A

RNG = np.random.default_rng(1234)


def _rand(*shape, mult=1.0):
    return RNG.standard_normal(shape) * mult


def _brute(q, k, v, scale, causal):
    """Scalar triple loop: exp, fsum, no numpy reductions."""
    N, d = q.shape
    dv = v.shape[1]
    o = np.zeros((N, dv))
    lse = np.zeros(N)
    for i in range(N):
        n = i + 1 if causal else k.shape[0]
        s = [scale * math.fsum(q[i, t] * k[j, t] for t in range(d)) for j in range(n)]
        r = max(s)
        e = [math.exp(x - r) for x in s]
        l = math.fsum(e)
        for c in range(dv):
            o[i, c] = math.fsum(e[j] * v[j, c] for j in range(n)) / l
        lse[i] = r + math.log(l)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 3), (2, 1), (5, 4), (8, 3)])
def test_brute_force_tiny(N, d, causal):
    q, k, v = _rand(N, d, mult=2.0), _rand(N, d, mult=2.0), _rand(N, d + 1)
    scale = 0.37
    o, lse = A.forward(q, k, v, scale, causal)
    ob, lb = _brute(q, k, v, scale, causal)
    assert np.abs(o - ob).max() <= 1e-13
    assert np.abs(lse - lb).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    B, H, N, d = 2, 3, 37, 16
    q, k, v = _rand(B, H, N, d), _rand(B, H, N, d), _rand(B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = A.forward(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    assert np.abs(o - ot.numpy()).max() <= 1e-12
    s = A.scores(q, k, scale, causal)
    assert np.abs(lse - logsumexp(s, axis=-1)).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd_float64(causal):
    B, H, N, d = 1, 2, 29, 8
    q, k, v, do = (_rand(B, H, N, d) for _ in range(4))
    scale = 0.3
    dq, dk, dv = A.backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    (ot * torch.from_numpy(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() <= 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_finite_differences(causal):
    N, d = 6, 3
    q, k, v, do = (_rand(N, d) for _ in range(4))
    scale = 0.8
    dq, dk, dv = A.backward(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        return float((A.forward(qq, kk, vv, scale, causal)[0] * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        fd = np.zeros_like(grad)
        for idx in np.ndindex(grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        rel = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-12)
        assert rel <= 1e-6, (which, rel)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    N, d = 12, 5
    q, v = _rand(N, d), _rand(N, d)
    k = np.tile(_rand(1, d), (N, 1))
    scale = 0.5
    o, lse = A.forward(q, k, v, scale, causal)
    s = scale * (q @ k[0])
    for i in range(N):
        n = i + 1 if causal else N
        assert np.allclose(o[i], v[:n].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[i] - (s[i] + math.log(n))) <= 1e-13
    meta = A.tie_metadata(q, k, v, scale, causal)
    expect = np.arange(1, N + 1) if causal else np.full(N, N)
    assert (meta["count"] == expect).all()


def test_single_dominant_key():
    N, d = 10, 4
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    j = 6
    q[:] = 0.0
    q[:, 0] = 1.0
    k[:, 0] = 0.0
    k[j, 0] = 80.0                       # score gap of 80 -> weight e^-80 elsewhere
    o, lse = A.forward(q, k, v, 1.0, False)
    assert np.abs(o - v[j]).max() <= 1e-15
    assert np.abs(lse - 80.0).max() <= 1e-14


def test_two_identical_dominant_keys_give_midpoint():
    N, d = 9, 3
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    q[:] = 0.0
    q[:, 1] = 1.0
    k[:, 1] = 0.0
    k[2, 1] = k[7, 1] = 70.0
    o, lse = A.forward(q, k, v, 1.0, False)
    assert np.abs(o - 0.5 * (v[2] + v[7])).max() <= 1e-14
    assert np.abs(lse - (70.0 + math.log(2.0))).max() <= 1e-13
    meta = A.tie_metadata(q, k, v, 1.0, False)
    assert (meta["count"] == 2).all()
    assert np.abs(meta["tie_mean"] - 0.5 * (v[2] + v[7])).max() <= 1e-15


def test_n_equals_one_and_causal_row_zero():
    q, k, v = _rand(1, 4), _rand(1, 4), _rand(1, 4)
    o, lse = A.forward(q, k, v, 0.5, False)
    assert np.array_equal(o, v)
    assert abs(lse[0] - 0.5 * float(q[0] @ k[0])) <= 1e-15
    q, k, v = _rand(7, 4), _rand(7, 4), _rand(7, 4)
    o, lse = A.forward(q, k, v, 0.5, True)
    assert np.array_equal(o[0], v[0])


def test_probability_rows_sum_to_one():
    q, k = _rand(3, 50, 8, mult=3.0), _rand(3, 50, 8, mult=3.0)
    for causal in (False, True):
        p, _ = A.probabilities(q, k, 0.35, causal)
        assert np.abs(p.sum(axis=-1) - 1.0).max() <= 1e-15 * 50
        if causal:
            assert (np.triu(p[0], 1) == 0).all()


def test_shift_invariance():
    """Softmax does not depend on the shift: adding a per-row constant to the
    scores (here through an extra key coordinate that every key shares)
    changes LSE by that constant and leaves O unchanged."""
    N, d = 16, 6
    q, k, v = _rand(N, d), _rand(N, d), _rand(N, d)
    shift = RNG.uniform(-30, 30, size=N)
    q2 = np.concatenate([q, shift[:, None]], axis=1)
    k2 = np.concatenate([k, np.ones((N, 1))], axis=1)
    o, lse = A.forward(q, k, v, 1.0, False)
    o2, lse2 = A.forward(q2, k2, v, 1.0, False)
    assert np.abs(o - o2).max() <= 1e-13
    assert np.abs((lse2 - lse) - shift).max() <= 1e-13
