"""fa_bwd_noalloc (the backward with its D vector in the library's fixed
per-device scratch) against fa_bwd, through the C ABI: two calls in a row,
the second on a smaller problem, each bitwise equal to fa_bwd on the same
inputs (same kernels, same arithmetic); and a problem past the scratch's
size is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

from gpu_util import random_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    import precision_numerics_fa_amd as fa
    assert torch.cuda.is_available()
    fa.load()
    return fa


def _case(fa, B, H, N, d, causal, seed):
    bits, dev = random_case(B, H, N, d, seed=seed, with_do=True)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, stabilize=True)
    return dev, o, lse


@pytest.mark.parametrize("first, second", [((2, 8, 1000, 128, True), (1, 3, 257, 64, False)),
                                           ((16, 16, 1024, 64, True), (1, 1, 77, 128, True))])
def test_noalloc_equals_fa_bwd_on_two_calls(fa, first, second):
    import torch
    for i, (B, H, N, d, causal) in enumerate((first, second)):
        say(f"noalloc call {i}: B={B} H={H} N={N} d={d} causal={causal}")
        dev, o, lse = _case(fa, B, H, N, d, causal, seed=100 + i + N)
        want = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal)
        got = fa.bwd_noalloc(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(a, b), (i, name)
            assert torch.isfinite(a.float()).all(), (i, name)


def test_noalloc_refuses_a_problem_past_its_scratch(fa):
    import torch
    lib = fa.load()
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    n = fa.NOALLOC_MAX_ROWS
    st = lib.fa_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, 1, n + 1, 64, 1, ctypes.c_float(0.125), 1, None)
    assert st == -6 and "scratch" in fa.status_string(st)
    torch.cuda.synchronize()
