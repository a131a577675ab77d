"""GPU parity of the split-key forward (fa_fwd_split, through the C ABI).

* With one range it is fa_fwd bit for bit (the partials and the merge add
  no rounding: every weight is 2^0).
* With several ranges (more ranges than key blocks included, so that some
  are empty) it meets the forward's gates against the exact oracle, and
  agrees with fa_fwd to the bit on nearly every output and within one bf16
  ulp (plus the FP32 rescaling allowance where a sum cancels) elsewhere: the
  replay of the earlier key blocks gives each range the one-pass running
  maximum and tie state, so the probabilities are rounded exactly as in one
  pass; only the FP32 rescalings are grouped differently.
* Rows whose maximum never repeats are bitwise the same with the fix on and
  off, and on the tie-heavy workload the fix removes the signed bias as it
  does in one pass.
"""
import numpy as np
import pytest

import fa_inputs as F
from oracle import metrics as Mt
from oracle import reference as REF

from gpu_util import device_inputs, head_f64, random_case, say, to_f64, LSE_TOL, lse_err

pytestmark = pytest.mark.gpu

MAX_ABS = 1.5e-2
MEAN_ABS = 2e-3


@pytest.fixture(scope="module")
def fa():
    import torch
    import precision_numerics_fa_amd as fa
    assert torch.cuda.is_available()
    fa.load()
    return fa


SHAPES = [(1, 1, 1, 64), (1, 2, 17, 64), (1, 1, 256, 64), (2, 1, 129, 128), (1, 3, 333, 128),
          (2, 2, 1000, 64), (1, 1, 640, 128)]


@pytest.mark.parametrize("stabilize", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_one_range_is_fa_fwd_bitwise(fa, B, H, N, d, causal, stabilize):
    say(f"split=1 B={B} H={H} N={N} d={d} causal={causal} stabilize={stabilize}")
    bits, dev = random_case(B, H, N, d, seed=N + 13 * d + B)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, stabilize=stabilize)
    o1, lse1 = fa.fwd_split(dev["q"], dev["k"], dev["v"], 1, causal=causal, stabilize=stabilize)
    assert np.array_equal(to_f64(o1), to_f64(o)) and np.array_equal(to_f64(lse1), to_f64(lse))


@pytest.mark.parametrize("splits", [2, 3, 5, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_split_against_oracle_and_fa_fwd(fa, B, H, N, d, causal, splits):
    say(f"split={splits} B={B} H={H} N={N} d={d} causal={causal}")
    bits, dev = random_case(B, H, N, d, seed=N + 7 * d + splits)
    scale = 1.0 / np.sqrt(d)
    for stabilize in (False, True):
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, stabilize=stabilize)
        os_, ls = fa.fwd_split(dev["q"], dev["k"], dev["v"], splits, causal=causal, stabilize=stabilize)
        q, k, v = (head_f64(bits[n]) for n in ("q", "k", "v"))
        o_ref, lse_ref = REF.forward(q, k, v, scale, causal)
        og, of = to_f64(os_), to_f64(o)
        e = Mt.output_errors(og, o_ref)
        assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS and e["finite"], e
        assert lse_err(to_f64(ls), lse_ref) <= LSE_TOL
        assert np.abs(to_f64(ls) - to_f64(lse)).max() <= 1e-5
        assert (og == of).mean() >= 0.98, (og == of).mean()
        # one bf16 ulp, plus 2^-20 |O_ref| row-wise for the regrouped FP32
        # rescalings where an output cancels to near zero
        bound = Mt.bf16_ulp(of) + 2.0 ** -20 * np.abs(o_ref).max(axis=-1, keepdims=True)
        assert (np.abs(og - of) <= bound).all()


def test_split_is_deterministic(fa):
    bits, dev = random_case(2, 3, 700, 128, seed=77)
    a = fa.fwd_split(dev["q"], dev["k"], dev["v"], 4, causal=True, stabilize=True)
    b = fa.fwd_split(dev["q"], dev["k"], dev["v"], 4, causal=True, stabilize=True)
    assert all(np.array_equal(to_f64(x), to_f64(y)) for x, y in zip(a, b))


def test_split_fix_touches_only_rows_with_a_repeated_maximum(fa):
    """The tie-heavy workload at reduced size, four ranges: rows that fa_fwd_diag
    reports as never shifted are bitwise equal between the fix on and off."""
    w = F.WORKLOADS["c2"].with_shape(B=2)
    full, dev = device_inputs(w)
    _, _, flags = fa.fwd_diag(dev["q"], dev["k"], dev["v"], causal=True, stabilize=True)
    on, lon = fa.fwd_split(dev["q"], dev["k"], dev["v"], 4, causal=True, stabilize=True)
    off, loff = fa.fwd_split(dev["q"], dev["k"], dev["v"], 4, causal=True, stabilize=False)
    untouched = to_f64(flags) == 0
    assert untouched.mean() > 0.5 and (~untouched).any()
    assert np.array_equal(to_f64(on)[untouched], to_f64(off)[untouched])
    assert np.array_equal(to_f64(lon)[untouched], to_f64(loff)[untouched])


def test_split_removes_the_tie_bias_like_one_pass(fa):
    """Q,K x4 (peaked scores), causal, 5% repeated-maximum rows, four ranges per
    query block (so most repeated maxima straddle a range boundary): the
    aligned signed error on tie rows drops with the fix as in one pass."""
    w = F.WORKLOADS["c2"].with_shape(B=4)
    full, dev = device_inputs(w)
    stats = {}
    for stabilize in (False, True):
        o, _ = fa.fwd_split(dev["q"], dev["k"], dev["v"], 4, causal=True, stabilize=stabilize)
        og = to_f64(o)
        d_all, s_all = [], []
        for b in range(w.B):
            q, k, v = (head_f64(full[n][b]) for n in ("q", "k", "v"))
            o_ref, _ = REF.forward(q, k, v, w.scale, True)
            meta = REF.tie_metadata(q, k, v, w.scale, True)
            tied = meta["count"] >= 2
            d_all.append((og[b] - o_ref)[tied])
            s_all.append(np.sign(o_ref - meta["tie_mean"])[tied])
        dd, ss = np.concatenate(d_all), np.concatenate(s_all)
        stats[stabilize] = ((dd * ss).mean(), (dd * ss).std(ddof=1) / np.sqrt(dd.size))
        say(f"  split tie rows aligned error stabilize={stabilize}: {stats[stabilize][0]:+.3e} "
            f"+- {stats[stabilize][1]:.1e}")
    assert stats[False][0] > 4 * stats[False][1]
    assert abs(stats[True][0]) < 0.5 * stats[False][0]


@pytest.mark.parametrize("splits", [2, 4])
def test_split_c4_full_sampled_heads(fa, splits):
    """Llama-2-7B shape (4, 32, 4096, 128), causal, fix on, at the range counts
    the sweep times: sampled heads against the exact oracle, and the whole
    output against fa_fwd."""
    import torch
    w = F.WORKLOADS["c4"]
    say(f"split c4 full splits={splits}")
    full, dev = device_inputs(w)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, stabilize=True)
    os_, ls = fa.fwd_split(dev["q"], dev["k"], dev["v"], splits, causal=True, stabilize=True)
    torch.cuda.synchronize()
    same = (os_ == o).float().mean().item()
    assert same >= 0.98, same
    assert (ls - lse).abs().max().item() <= 1e-5
    for b, h in F.sample_pairs(w, 2, seed=splits):
        q, k, v = (head_f64(full[n][b, h]) for n in ("q", "k", "v"))
        o_ref, _ = REF.forward(q, k, v, w.scale, True)
        e = Mt.output_errors(to_f64(os_[b, h]), o_ref)
        assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS, (b, h, e)
