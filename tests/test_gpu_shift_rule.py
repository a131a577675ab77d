"""GPU checks of the repeated-maximum shift (page 2, "Mechanism 2": detect a
row maximum that occurs more than once and move the softmax shift so that
the exponent at the maximum is strictly below 1).

* The hand-derived worked example (tests/golden/tie_midpoint.json) runs
  through fa_fwd at both head sizes: an output on an exact bf16 rounding
  midpoint stays there with the fix off (1.0) and leaves it with the fix on
  (1.0078125); the same with a negative maximum; and a maximum large enough
  that the shift is folded.  O is compared bit for bit.  The shift itself is
  read back from fa_fwd_split's workspace (with one key range its M part
  holds every row's final shift) and compared bit for bit with the example's
  values: a fold by whole multiples of 32 changes neither O nor LSE, so only
  the shift shows it.
* Its binary16 counterpart (tie_midpoint_f16.json) runs through fa_fwd_ex.
* Against the blocked emulation (oracle B) at the kernel's key block, on the
  tie-heavy workloads: the rows the kernel flags as shifted are exactly the
  rows the emulation shifts, and outputs agree bitwise on shifted and
  unshifted rows alike, gated separately.
* The aligned signed error left on tie rows with the fix on is the
  emulation's own (the reading of the rule, not the kernel).
"""
import json
import os

import numpy as np
import pytest

import fa_inputs as F
from oracle import emulation as EMU
from oracle import metrics as Mt
from oracle import reference as REF

from gpu_util import device_inputs, head_f64, say, to_f64

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def fa():
    import torch
    import precision_numerics_fa_amd as fa
    assert torch.cuda.is_available()
    fa.load()
    return fa


def _padded(rows, d, dtype):
    """(1, 1, len(rows), d) tensor whose first column holds `rows` (16-bit
    exact values) and whose other columns are 0."""
    import torch
    t = torch.zeros((1, 1, len(rows), d), dtype=dtype)
    t[0, 0, :, 0] = torch.tensor(rows, dtype=torch.float64).to(dtype)
    return t.cuda()


def _split_shift(fa, q, k, v, stabilize):
    """fa_fwd_split with one key range; returns (O, LSE, M), M the per-row
    final shift from the workspace (layout in fa.h: O_bar, then l, then M,
    each at a 256-byte boundary)."""
    import torch
    B, H, N, d = q.shape
    ws = torch.zeros(fa.fwd_split_workspace_bytes(B, H, N, d, 1), dtype=torch.uint8, device=q.device)
    o, lse = fa.fwd_split(q, k, v, 1, causal=False, scale=1.0, stabilize=stabilize, workspace=ws)
    torch.cuda.synchronize()
    r256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    ob, vb = r256(B * H * N * d * 4), r256(B * H * N * 4)
    m = ws[ob + vb: ob + vb + B * H * N * 4].view(torch.float32).cpu().numpy()
    return o, lse, m


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ["plain", "negative", "folded"])
def test_golden_tie_midpoint_through_fa_fwd(fa, d, case):
    import torch
    g = json.load(open(os.path.join(GOLDEN, "tie_midpoint.json")))
    say(f"golden tie midpoint through fa_fwd: d={d} case={case}")
    qv = {"plain": 1.0, "negative": -1.0, "folded": 1.0}[case]
    kv = g["fold_k"][0][0] if case == "folded" else g["k"][0][0]
    pre = {"plain": "", "negative": "neg_", "folded": "fold_"}[case]
    # two query rows (the example's query twice), two identical keys
    q = _padded([qv, qv], d, torch.bfloat16)
    k = _padded([kv, kv], d, torch.bfloat16)
    v = _padded([g["v"][0][0], g["v"][1][0]], d, torch.bfloat16)
    lse_exact = g[pre + "lse"] if pre else g["lse"]
    for stab, suffix in ((False, "fix_off"), (True, "fix_on")):
        o, lse = fa.fwd(q, k, v, causal=False, scale=1.0, stabilize=stab)
        o_expect = g[pre + "o_" + suffix] if case == "folded" else g["o_" + suffix]
        of = to_f64(o[0, 0])
        assert (of[:, 0] == o_expect).all(), (stab, of[:, 0], o_expect)
        assert (of[:, 1:] == 0.0).all()
        assert np.abs(to_f64(lse[0, 0]) - lse_exact).max() <= 4e-6 * max(1.0, abs(lse_exact))
        o_s, lse_s, m = _split_shift(fa, q, k, v, stab)
        assert torch.equal(o_s, o) and torch.equal(lse_s, lse)
        assert (m == np.float32(g[pre + "M_" + suffix])).all(), (stab, m, g[pre + "M_" + suffix])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_golden_tie_midpoint_f16_through_fa_fwd_ex(fa, d, sign):
    import torch
    g = json.load(open(os.path.join(GOLDEN, "tie_midpoint_f16.json")))
    say(f"golden binary16 tie midpoint through fa_fwd_ex: d={d} sign={sign}")
    q = _padded([sign * g["q"][0][0]] * 2, d, torch.float16)
    k = _padded([g["k"][0][0], g["k"][1][0]], d, torch.float16)
    v = _padded([g["v"][0][0], g["v"][1][0]], d, torch.float16)
    lse_exact = g["lse"] if sign > 0 else g["lse"] - 4.0
    for stab, key in ((False, "o_fix_off"), (True, "o_fix_on")):
        o, lse = fa.fwd_ex(q, k, v, causal=False, scale=1.0, stabilize=stab)
        of = to_f64(o[0, 0])
        assert (of[:, 0] == g[key]).all(), (stab, of[:, 0], g[key])
        assert (of[:, 1:] == 0.0).all()
        assert np.abs(to_f64(lse[0, 0]) - lse_exact).max() <= 4e-6


def _emulation_agreement(fa, w, heads):
    """Per variant: flag agreement with the emulation, and bitwise agreement /
    worst ulp distance of O on the shifted and on the unshifted rows."""
    full, dev = device_inputs(w)
    bk = fa.fwd_tile(w.d)[1]
    out = {}
    for stab in (False, True):
        o, _, flags = fa.fwd_diag(dev["q"], dev["k"], dev["v"], causal=w.causal, stabilize=stab)
        of, fl = to_f64(o), flags.cpu().numpy().astype(bool)
        acc = {"flag_mismatch": 0, "rows": 0, "shifted": [0, 0, 0.0], "unshifted": [0, 0, 0.0]}
        for (b, h) in heads:
            q, k, v = (head_f64(full[n][b, h]) for n in ("q", "k", "v"))
            ob, _, st = EMU.forward(q, k, v, w.scale, w.causal, block=bk, stabilize=stab, return_state=True)
            acc["flag_mismatch"] += int((st["ever_shifted"] != fl[b, h]).sum())
            acc["rows"] += w.N
            for name, sel in (("shifted", fl[b, h]), ("unshifted", ~fl[b, h])):
                a, e = of[b, h][sel], ob[sel]
                s = acc[name]
                s[0] += int((a == e).sum())
                s[1] += a.size
                if a.size:
                    # in ulps of each row's largest |O| (an element near zero after
                    # cancellation differs by tiny absolute amounts that are many
                    # ulps of its own size)
                    scale = Mt.bf16_ulp(np.abs(e).max(axis=-1, keepdims=True))
                    s[2] = max(s[2], float((np.abs(a - e) / scale).max()))
        out[stab] = acc
    return out


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_shifted_and_unshifted_rows_match_the_emulation(fa, name):
    """The kernel shifts exactly the rows the emulation shifts, and its
    outputs equal the emulation's bit for bit on at least 99% of the elements
    of each kind of row, and elsewhere within one bf16 ulp of the row's
    largest output (MFMA summation order and the hardware exp2 differ from
    the CPU's)."""
    w = F.WORKLOADS[name]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    say(f"{name}: emulation agreement on {len(heads)} heads")
    res = _emulation_agreement(fa, w, heads)
    for stab, acc in res.items():
        say(f"  stabilize={stab}: flag mismatches {acc['flag_mismatch']} of {acc['rows']} rows; "
            + "; ".join(f"{k} {s[0] / max(s[1], 1):.5f} bitwise of {s[1]}, max {s[2]:.1f} ulp"
                        for k, s in ((k, acc[k]) for k in ("shifted", "unshifted"))))
        assert acc["flag_mismatch"] <= acc["rows"] // 1000
        if not stab:
            assert acc["shifted"][1] == 0
        for kind in ("shifted", "unshifted"):
            same, n, ulps = acc[kind]
            if n:
                assert same >= 0.99 * n, (stab, kind, same / n)
                assert ulps <= 1.0, (stab, kind, ulps)
    assert res[True]["shifted"][1] > 0


def test_tie_bias_left_with_the_fix_is_the_emulations(fa):
    """On every head of the tie-heavy workload (Q,K x4, 5% repeated-max rows)
    the aligned signed error on tie rows is measured for the kernel and for
    the emulation at the kernel's key block, on the same rows: with the fix
    off both show the directional bias, with it on both lose most of it, and
    the two agree to well within the statistic's own standard error."""
    w = F.WORKLOADS["c2"]
    full, dev = device_inputs(w)
    bk = fa.fwd_tile(w.d)[1]
    res = {}
    for stab in (False, True):
        o, _ = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, stabilize=stab)
        of = to_f64(o)
        gd, ed, sg = [], [], []
        for b in range(w.B):
            for h in range(w.H):
                q, k, v = (head_f64(full[n][b, h]) for n in ("q", "k", "v"))
                o_ref, _ = REF.forward(q, k, v, w.scale, True)
                meta = REF.tie_metadata(q, k, v, w.scale, True)
                tied = meta["count"] >= 2
                ob, _ = EMU.forward(q, k, v, w.scale, True, block=bk, stabilize=stab)
                gd.append((of[b, h] - o_ref)[tied])
                ed.append((ob - o_ref)[tied])
                sg.append(np.sign(o_ref - meta["tie_mean"])[tied])
        g_al, e_al, s = (np.concatenate(x) for x in (gd, ed, sg))
        g_al, e_al = g_al * s, e_al * s
        se = e_al.std(ddof=1) / np.sqrt(e_al.size)
        res[stab] = (g_al.mean(), e_al.mean(), se)
        say(f"  c2 stabilize={stab}: aligned tie error kernel {g_al.mean():+.3e}, emulation {e_al.mean():+.3e} "
            f"(se {se:.1e}, {g_al.size} elements)")
        assert abs(g_al.mean() - e_al.mean()) <= 0.5 * se
    assert res[False][1] > 10 * res[False][2]
    assert abs(res[True][0]) < 0.25 * res[False][0]
