"""The seeded workload generator: reproducibility, shapes, and the
repeated-maximum construction (confirmed with the exact oracle)."""
import numpy as np
import pytest
import torch

import fa_inputs as F
from oracle import reference as A


def test_bf16_encoding_matches_torch():
    x = np.random.default_rng(0).standard_normal(50000).astype(np.float32) * 7
    bits = F.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = F.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_heads_are_reproducible_and_distinct():
    w = F.WORKLOADS["c2"].with_shape(N=128)
    a = F.head(w, 1, 2)
    b = F.head(w, 1, 2)
    c = F.head(w, 2, 1)
    for n in ("q", "k", "v"):
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])


def test_full_tensor_is_concatenation_of_heads():
    w = F.WORKLOADS["c5"].with_shape(B=2, H=3, N=64)
    full = F.full(w)
    for (b, h) in [(0, 0), (1, 2)]:
        hd = F.head(w, b, h)
        for n in ("q", "k", "v", "do"):
            assert np.array_equal(full[n][b, h], hd[n])
        assert np.array_equal(full["tie_rows"][(b, h)], hd["tie_rows"])


@pytest.mark.parametrize("name,pairs", [("c1", [(0, 0)]), ("c2", [(0, 0), (5, 7)]), ("c5", [(3, 9)])])
def test_repeated_max_rows_confirmed_by_exact_oracle(name, pairs):
    w = F.WORKLOADS[name]
    target = int(round(w.tie_frac * w.N))
    for (b, h) in pairs:
        hd = F.head(w, b, h)
        q, k, v = (F.bf16_bits_to_f32(hd[n]).astype(np.float64) for n in ("q", "k", "v"))
        meta = A.tie_metadata(q, k, v, w.scale, w.causal)
        tied = np.flatnonzero(meta["count"] >= 2)
        assert np.array_equal(tied, hd["tie_rows"])
        assert len(tied) >= target
        if w.causal:
            assert 0 not in tied


def test_lowrank_component_is_shared():
    w = F.WORKLOADS["c3"].with_shape(N=256)
    a, b = F.head(w, 0, 0), F.head(w, 3, 5)
    ka = F.bf16_bits_to_f32(a["k"]).astype(np.float64)
    kb = F.bf16_bits_to_f32(b["k"]).astype(np.float64)
    fa, fb = F._lowrank_factors(w)
    common = 0.5 * (fa @ fb.T) / 2.0
    # removing the shared rank-4 term leaves residuals with ~unit variance
    for kk in (ka, kb):
        r = kk - common
        assert 0.8 < r.std() < 1.2
    assert abs(np.corrcoef(ka.ravel(), kb.ravel())[0, 1] - 0.2) < 0.05


def test_sample_pairs():
    w = F.WORKLOADS["c3"]
    p = F.sample_pairs(w, 32)
    assert len(p) == 32 and len(set(p)) == 32
    assert p == F.sample_pairs(w, 32)
    assert all(0 <= b < w.B and 0 <= h < w.H for b, h in p)
