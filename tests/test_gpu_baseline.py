"""GPU parity of the unfused FP32-accumulating baseline (fa_base_*, through the
C ABI) against the CPU oracle.

* Each step is checked on its own where its result is exact: the score
  kernel on integer-valued inputs (every dot product exact in FP32, so S must
  equal fl32(t * scale) bit for bit on every entry the softmax reads); the PV
  kernel on probabilities and values whose products and sums are exact.
* The softmax step, fed the GPU's own S, against the baseline emulation's
  softmax of the same S: its row sum is reduced in a different order, so a
  few probabilities may land one bf16 ulp away; the rest are bit-identical,
  and P is zero on every key past the row's last visible one that the PV
  step reads.
* The whole baseline against the exact oracle (the forward's gates) and
  against the baseline emulation, on ragged shapes; at full Llama-2-7B shape
  on sampled heads.
* The hand-derived three-way-tie example: the baseline's bf16(1/3)
  probabilities give 2.34375 where FlashAttention (fix off or on) gives the
  correctly rounded 2.328125.
"""
import json
import os

import numpy as np
import pytest

import fa_inputs as F
from oracle import baseline as BASE
from oracle import emulation as EMU
from oracle import metrics as Mt
from oracle import reference as REF

from gpu_util import device_inputs, head_f64, random_case, say, to_dev, to_f64, LSE_TOL, lse_err

pytestmark = pytest.mark.gpu

MAX_ABS = 1.5e-2
MEAN_ABS = 2e-3
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def fa():
    import torch
    import precision_numerics_fa_amd as fa
    assert torch.cuda.is_available()
    fa.load()
    return fa


def _visible(N, causal):
    return np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)


def _pv_read_width(N, ld, causal):
    """Per row, the keys the PV step reads: to the end of the row's 64-key
    block (causal) or the whole padded row."""
    if not causal:
        return np.full(N, ld)
    return np.minimum(ld, 64 * (np.arange(N) // 64 + 1))


SHAPES = [(1, 1, 1, 64), (1, 2, 17, 64), (2, 1, 129, 128), (1, 3, 200, 64), (2, 2, 333, 128), (1, 1, 64, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_scores_exact_on_integer_inputs(fa, B, H, N, d, causal):
    import torch
    say(f"base scores B={B} H={H} N={N} d={d} causal={causal}")
    rng = np.random.default_rng(N * 3 + d)
    qi = rng.integers(-3, 4, (B, H, N, d)).astype(np.float32)
    ki = rng.integers(-3, 4, (B, H, N, d)).astype(np.float32)
    q = torch.from_numpy(qi).to(torch.bfloat16).cuda()
    k = torch.from_numpy(ki).to(torch.bfloat16).cuda()
    scale = 1.0 / np.sqrt(d)
    s = fa.base_scores(q, k, causal=causal, scale=scale)
    torch.cuda.synchronize()
    s = s.cpu().numpy().astype(np.float64)[..., :N]
    ref = BASE.scores(qi.astype(np.float64), ki.astype(np.float64), scale, causal)
    vis = np.broadcast_to(_visible(N, causal), ref.shape)
    assert np.array_equal(s[vis], ref[vis])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_softmax_against_emulation_on_the_same_scores(fa, B, H, N, d, causal):
    import torch
    say(f"base softmax B={B} H={H} N={N} d={d} causal={causal}")
    bits, dev = random_case(B, H, N, d, seed=N + 5 * d + B, mult=2.0)
    s = fa.base_scores(dev["q"], dev["k"], causal=causal)
    p, lse = fa.base_softmax(s, causal=causal)
    torch.cuda.synchronize()
    ld = fa.base_ld(N)
    s_host = s.cpu().numpy().astype(np.float64)[..., :N]
    s_host = np.where(_visible(N, causal), s_host, -np.inf)
    p_ref, lse_ref = BASE.softmax(s_host)
    p_gpu = to_f64(p)
    width = _pv_read_width(N, ld, causal)
    cols = np.arange(ld)[None, :]
    written = (cols < width[:, None])[:, :N]      # P past the PV step's read range is not written
    pg = p_gpu[..., :N][..., written]
    pr = p_ref[..., written]
    assert np.isfinite(pg).all()
    assert (pg == pr).mean() >= 0.99, (pg == pr).mean()
    assert (np.abs(pg - pr) <= Mt.bf16_ulp(pr)).all()
    last_visible = np.arange(N) + 1 if causal else np.full(N, N)
    beyond = (cols >= last_visible[:, None]) & (cols < width[:, None])
    assert (p_gpu[..., beyond] == 0).all()
    assert np.abs(to_f64(lse) - lse_ref).max() <= 2e-6 * max(1.0, np.abs(lse_ref).max())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES)
def test_pv_exact_on_exact_products(fa, B, H, N, d, causal):
    """P entries are multiples of 1/64 below 1 and V entries small integers:
    every product and partial sum is exact in FP32, so O = bf16(P V) exactly."""
    import torch
    say(f"base pv B={B} H={H} N={N} d={d} causal={causal}")
    ld = fa.base_ld(N)
    rng = np.random.default_rng(N + d + 11)
    p = rng.integers(0, 64, (B, H, N, ld)).astype(np.float32) / 64.0
    width = _pv_read_width(N, ld, causal)
    vis = np.zeros((N, ld), dtype=bool)
    vis[:, :N] = _visible(N, causal)
    p = np.where(vis, p, 0.0).astype(np.float32)
    p_pad = np.where(np.arange(ld)[None, :] < width[:, None], p, np.float32(7.0))  # never read
    v = rng.integers(-4, 5, (B, H, N, d)).astype(np.float32)
    o = fa.base_pv(torch.from_numpy(p_pad).to(torch.bfloat16).cuda(), torch.from_numpy(v).to(torch.bfloat16).cuda(),
                   causal=causal)
    torch.cuda.synchronize()
    ref = EMU.bf16(p[..., :N].astype(np.float64) @ v.astype(np.float64))
    assert np.array_equal(to_f64(o), ref)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d", SHAPES + [(1, 2, 1000, 128), (2, 2, 511, 64)])
def test_baseline_against_oracles(fa, B, H, N, d, causal):
    import torch
    say(f"base fwd B={B} H={H} N={N} d={d} causal={causal}")
    bits, dev = random_case(B, H, N, d, seed=3 * N + d + B)
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.base_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    q, k, v = (head_f64(bits[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = REF.forward(q, k, v, scale, causal)
    og = to_f64(o)
    e = Mt.output_errors(og, o_ref)
    assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS and e["finite"], e
    assert lse_err(to_f64(lse), lse_ref) <= LSE_TOL
    o_emu, _ = BASE.forward(q, k, v, scale, causal)
    assert (og == o_emu).mean() >= 0.97, (og == o_emu).mean()
    # the three steps through their own entry points compose to fa_base_fwd
    # bit for bit, and the PV step on the GPU's own P is the FP32-accumulated
    # product to one bf16 ulp (the summation order is the only difference;
    # against the emulation's P a probability one ulp apart can move O by more)
    s_ = fa.base_scores(dev["q"], dev["k"], causal=causal)
    # P past the read range is never written: start from zeros, so that no
    # uninitialised device memory is converted below
    p_, _ = fa.base_softmax(s_, causal=causal, p=torch.zeros((B, H, N, fa.base_ld(N)), dtype=torch.bfloat16,
                                                              device=s_.device))
    o2 = fa.base_pv(p_, dev["v"], causal=causal)
    assert np.array_equal(to_f64(o2), og)
    p_read = np.where(_visible(N, causal), to_f64(p_)[..., :N], 0.0)   # P past the read range is not written
    pv_ref = EMU.bf16(EMU.fl32(p_read @ v))
    # one bf16 ulp of the result, plus an FP32 accumulation allowance of 2^-20
    # times sum |P| |V| (it matters only where the sum cancels to near zero)
    bound = Mt.bf16_ulp(pv_ref) + 2.0 ** -20 * (np.abs(p_read) @ np.abs(v))
    assert (np.abs(og - pv_ref) <= bound).all()


def test_golden_three_way_tie_on_gpu(fa):
    import torch
    with open(os.path.join(GOLDEN, "baseline_three_way_tie.json")) as f:
        g = json.load(f)
    d = 64
    pad = lambda a: np.pad(np.array(a, dtype=np.float32), ((0, 0), (0, d - len(a[0]))))[None, None]  # noqa: E731
    q, k, v = (torch.from_numpy(pad(g[n])).to(torch.bfloat16).cuda() for n in ("q", "k", "v"))
    q = q.expand(1, 1, 3, d).contiguous()   # three queries, all seeing the three tied keys
    o, lse = fa.base_fwd(q, k, v, causal=False, scale=g["scale"])
    og = to_f64(o)[0, 0]
    assert (og[:, :2] == np.array(g["o_baseline"])).all() and (og[:, 2:] == 0).all()
    assert np.abs(to_f64(lse) - g["lse"]).max() < 1e-6
    for stab in (False, True):
        o_fa, _ = fa.fwd(q, k, v, causal=False, scale=g["scale"], stabilize=stab)
        assert (to_f64(o_fa)[0, 0, :, :2] == np.array(g["o_flash"])).all()


@pytest.mark.parametrize("stabilize", [False, True])
def test_c4_full_baseline_and_flash_on_sampled_heads(fa, stabilize):
    """Llama-2-7B shape (4, 32, 4096, 128), causal: the baseline and
    FlashAttention in the launch configuration the benchmark times, both
    against the exact oracle on seeded heads."""
    import torch
    w = F.WORKLOADS["c4"]
    say(f"base c4 full stabilize={stabilize}")
    full, dev = device_inputs(w)
    o_b, _ = fa.base_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    o_f, _ = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, stabilize=stabilize)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(w.d)
    for b, h in F.sample_pairs(w, 3, seed=int(stabilize) + 7):
        q, k, v = (head_f64(full[n][b, h]) for n in ("q", "k", "v"))
        o_ref, _ = REF.forward(q, k, v, scale, True)
        for name, o in (("baseline", o_b), ("flash", o_f)):
            e = Mt.output_errors(to_f64(o[b, h]), o_ref)
            assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS, (name, b, h, e)


def test_mfma_probe_counts_its_flop_and_computes_the_product(fa):
    """The MFMA ceiling probe: the FLOP it reports, and its result against the
    product its operands define (small exact values, so bit-exact), which also
    checks the operand and accumulator layouts documented in fa_device.hpp."""
    import torch
    blocks, iters = 8, 3
    flop, out = fa.mfma_probe(blocks, iters)
    torch.cuda.synchronize()
    assert flop == blocks * 4 * iters * 8 * 2 * 32 * 32 * 16
    lanes = np.arange(64)
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for l in lanes:
        for j in range(8):
            A[l % 32, 8 * (l // 32) + j] = ((l + j) & 7) / 1024.0
            Bm[8 * (l // 32) + j, l % 32] = ((3 * l + j) & 7) / 1024.0
    C = iters * (A @ Bm)
    expect = np.array([sum(C[8 * (t // 4) + 4 * (l // 32) + t % 4, l % 32] for t in range(8)) for l in lanes])
    got = out.cpu().numpy().astype(np.float64).reshape(blocks * 4, 64)
    assert np.array_equal(got, np.broadcast_to(expect, got.shape))


def test_issue_probe_runs_every_kind(fa):
    """The instruction-issue probe: every kind at one and two waves per SIMD
    launches and completes.  For the MFMA kind (small exact operands) the
    output of the active waves grows with the iteration count by the product
    its operands define, and that of the idle waves does not change: only the
    requested waves run the loop.  The LDS-read kind adds the fold of the
    chunks it read, computed here from the values the kernel stores."""
    import torch
    blocks = 8
    for kind in range(len(fa.ISSUE_PROBE_KINDS)):
        for w in (1, 2):
            if kind == 7 and w == 1:
                continue
            print(f"issue probe kind {kind} ({fa.ISSUE_PROBE_KINDS[kind]}) waves/SIMD {w}", flush=True)
            fa.issue_probe(kind, w, blocks, 3)
            torch.cuda.synchronize()
    for w in (1, 2):
        o3 = fa.issue_probe(0, w, blocks, 3).cpu().numpy().astype(np.float64).reshape(blocks, 8, 64)
        o6 = fa.issue_probe(0, w, blocks, 6).cpu().numpy().astype(np.float64).reshape(blocks, 8, 64)
        diff = o6 - o3
        active, idle = diff[:, : 4 * w], diff[:, 4 * w :]
        # every accumulator entry is sum_k a_k b_k = -0.064453125 (a = (j+1)/64,
        # b = (1-j)/64 over both k halves); three more iterations of two MFMAs
        # on each of four accumulators of 16 entries add 6 * 64 of them, up to
        # the float rounding of each thread's total
        assert np.allclose(active, 6 * 64 * -0.064453125, atol=1e-2), (w, active.min(), active.max())
        assert np.all(idle == 0), w
    # the LDS-read kind folds (xor) the 16-byte chunks it reads; the chunks
    # hold the bf16 pairs ((i mod 64) / 256, -(i mod 32) / 256) for 32-bit word
    # i, and iteration `it` of thread t reads chunks (t + 512 r + 67 it) mod
    # 4096, r < 8; the low byte of the fold is added to the output
    i = np.arange(16384)
    bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint32)  # noqa: E731
    words = (bits(-(i % 32) / 256.0) << 16) | bits((i % 64) / 256.0)
    chunk = np.bitwise_xor.reduce(words.reshape(4096, 4), axis=1)
    tid = np.arange(512)

    def fold(iters):
        xr = np.zeros(512, dtype=np.uint32)
        for it in range(iters):
            for r in range(8):
                xr ^= chunk[(tid + 512 * r + 67 * it) & 4095]
        return (xr & 255).astype(np.float64)

    for w in (1, 2):
        o3 = fa.issue_probe(8, w, blocks, 3).cpu().numpy().astype(np.float64).reshape(blocks, 512)
        o6 = fa.issue_probe(8, w, blocks, 6).cpu().numpy().astype(np.float64).reshape(blocks, 512)
        expect = np.where(tid < 256 * w, fold(6) - fold(3), 0.0)
        assert np.allclose(o6 - o3, np.broadcast_to(expect, o6.shape), atol=1e-3), w


def test_hbm_probe_reads_every_word(fa):
    """The read probe folds (xor) each thread's words: the xor over all sink
    values equals the xor of the whole buffer, including a tail shorter than
    the grid stride."""
    import torch
    for n in (1 << 20, 12, 4096 * 256 * 4 * 3 + 40):
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda")
        sink = fa.hbm_probe(src)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, n


@pytest.mark.parametrize("causal", [False, True])
def test_baseline_at_its_longest_rows(fa, causal):
    """N = 16384, the longest row the baseline's softmax holds in registers
    (one head of each head size): sampled rows against the exact oracle row
    by row, and the last rows of the tail."""
    import torch
    N = 16384
    for d in (64, 128):
        say(f"base longest rows N={N} d={d} causal={causal}")
        bits, dev = random_case(1, 1, N, d, seed=91 + d + int(causal))
        scale = 1.0 / np.sqrt(d)
        o, lse = fa.base_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        torch.cuda.synchronize()
        q, k, v = (head_f64(bits[n])[0, 0] for n in ("q", "k", "v"))
        rows = np.concatenate([np.random.default_rng(d).choice(N, 24, replace=False), [0, 63, 64, N - 2, N - 1]])
        og, lg = to_f64(o)[0, 0], to_f64(lse)[0, 0]
        for i in rows:
            L = i + 1 if causal else N
            o_ref, lse_ref = REF.forward(q[i:i + 1], k[:L], v[:L], scale, False)
            assert np.abs(og[i] - o_ref[0]).max() <= 1.5e-2, i
            assert lse_err(lg[i], lse_ref[0]) <= LSE_TOL, i
