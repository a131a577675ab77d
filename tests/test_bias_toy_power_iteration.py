"""The bias toy's spectral norms come from power iteration: pinned against
the singular values numpy computes (a library routine of a different
algorithm) on matrices with a known gap, and against a closed form."""
import numpy as np
import torch

from precision_numerics_fa_amd.bias_toy import spectral_norm


def test_power_iteration_matches_the_largest_singular_value():
    rng = np.random.default_rng(3)
    for n in (8, 64):
        W = torch.from_numpy(rng.standard_normal((n, n)))
        s_ref = float(np.linalg.svd(W.numpy(), compute_uv=False)[0])
        v = torch.ones(n, dtype=torch.float64) / n ** 0.5
        s, v = spectral_norm(W, v, 200)
        assert abs(s - s_ref) <= 1e-9 * s_ref
        # warm start: a few more steps from the converged vector change nothing
        s2, _ = spectral_norm(W, v, 3)
        assert abs(s2 - s_ref) <= 1e-9 * s_ref


def test_power_iteration_closed_form():
    # diag(3, 1) rotated: sigma_max = 3 exactly
    c, s_ = np.cos(0.3), np.sin(0.3)
    R = np.array([[c, -s_], [s_, c]])
    W = torch.from_numpy(R @ np.diag([3.0, 1.0]) @ R.T)
    s, _ = spectral_norm(W, torch.tensor([1.0, 0.0], dtype=torch.float64), 60)
    assert abs(s - 3.0) <= 1e-12
