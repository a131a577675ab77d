"""Largest sizes: tensors of more than 2^31 elements, so that head offsets
need 64-bit arithmetic in every kernel (forward, row-dot, dK/dV, dQ).

(B, H, N, d) = (1, 264, 65536, 128), causal: 2.2e9 elements, 4.4 GB per
tensor.  The heads are copies of four distinct seeded heads (head h holds
base head h % 4), placed by PyTorch device copies.  Two checks:

* properties that hold at any size: every head equals, bit for bit, its copy
  at the start of the tensor (heads past element 2^31 included), in O, LSE,
  dQ, dK and dV;
* the oracle, row by row, on sampled rows of the last head (whose every
  element lies past 2^31): a causal row i is plain softmax attention over keys
  0..i, which the exact oracle computes in O(N d).
"""
import numpy as np
import pytest

import fa_inputs as F
from oracle import metrics as Mt
from oracle import reference as REF

from gpu_util import LSE_TOL, lse_err, say, to_f64

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 264, 65536, 128
NBASE = 4


@pytest.fixture(scope="module")
def big():
    import torch
    import precision_numerics_fa_amd as fa
    assert torch.cuda.is_available()
    assert B * H * N * D > 2 ** 31
    say(f"large: building (B,H,N,d)=({B},{H},{N},{D}) from {NBASE} seeded heads")
    base = {n: F.random_bf16((NBASE, N, D), 7000 + i) for i, n in enumerate(("q", "k", "v", "do"))}
    dev = {}
    for n, bits in base.items():
        blk = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        t = torch.empty((B, H, N, D), dtype=torch.bfloat16, device="cuda")
        t.view(H // NBASE, NBASE, N, D).copy_(blk.unsqueeze(0).expand(H // NBASE, NBASE, N, D))
        dev[n] = t
        del blk
    torch.cuda.synchronize()
    return fa, base, dev


def test_large_forward_copies_and_sampled_rows(big):
    import torch
    fa, base, dev = big
    say("large: forward")
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, stabilize=True)
    torch.cuda.synchronize()
    ov = o.view(H // NBASE, NBASE, N, D)
    lv = lse.view(H // NBASE, NBASE, N)
    for g in (1, H // NBASE // 2, H // NBASE - 1):
        assert torch.equal(ov[g], ov[0]) and torch.equal(lv[g], lv[0]), g
    last = H - 1
    q, k, v = (F.bf16_bits_to_f32(base[n][last % NBASE]).astype(np.float64) for n in ("q", "k", "v"))
    scale = 1.0 / np.sqrt(D)
    rows = [0, 1, 4095, 33333, N - 1000, N - 2, N - 1]
    og, lg = to_f64(o[0, last]), lse[0, last].double().cpu().numpy()
    for i in rows:
        orf, lrf = REF.forward(q[i:i + 1], k[:i + 1], v[:i + 1], scale, False)
        e = Mt.output_errors(og[i:i + 1], orf)
        assert e["max_abs"] <= 1.5e-2, (i, e)
        assert lse_err(lg[i], lrf[0]) <= LSE_TOL, (i, lg[i], lrf[0])
    say("large: forward ok")


def test_large_backward_copies(big):
    import torch
    fa, base, dev = big
    say("large: backward")
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, stabilize=True)
    dq, dk, dv = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        tv = t.view(H // NBASE, NBASE, N, D)
        for g in (1, H // NBASE - 1):
            assert torch.equal(tv[g], tv[0]), (name, g)
        assert bool(torch.isfinite(tv[-1]).all()), name
    say("large: backward ok")
