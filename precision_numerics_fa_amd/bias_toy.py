"""Bias accumulation in a toy attention layer, through fa_fwd / fa_bwd.

Page 2 ("Mechanism 1" and "Mechanism 2"): a rounding error that is not zero
mean -- the one a repeated row maximum causes in the BF16 probabilities --
meets similar low-rank update directions step after step, so it adds up in
the weights instead of averaging out, and the spectral norms of W_Q and W_K
drift.  This module runs that experiment at toy scale on synthetic data (no
model, no dataset):

* one attention head, d = 64; every step draws a fresh batch of B sequences
  of N tokens whose inputs are low rank (a shared component, rank-r
  structure, 10% noise);
* queries and values read the token input, keys read a key input that
  equals it except at two "sink" positions per sequence, which carry one
  fixed large vector: their keys are identical and their values are not, so
  rows whose attention they dominate tie at the row maximum.  The untied
  control gives the second sink a key input 1% away (no ties, the same
  attention mass);
* q = x W_Q, k = a W_K, v = x W_V, rounded to bf16; the loss is the mean
  squared distance of the attention output to a fixed linear map of x.

Along a float32 reference trajectory (SGD on float32 gradients of the same
bf16 q, k, v), the W_Q, W_K, W_V gradients through the library (fix off and
fix on) are compared at every step, and each variant also trains on its own
gradients.  Recorded per step: the spectral norms of W_Q and W_K of the
reference and of each trained variant, and the spectral norm of the
accumulated gradient error sum_t (g_t - g_ref,t) of W_Q and W_K, which grows
like t when the error keeps one direction and like sqrt(t) when it does not.
Spectral norms come from power iteration, warm-started from the previous
step's vector.

Run:  python -m precision_numerics_fa_amd.bias_toy [--steps 300] [--out f.json]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import sys
from typing import Dict, List, Optional

NAMES = ("W_Q", "W_K", "W_V")


@dataclasses.dataclass(frozen=True)
class ToyConfig:
    B: int = 8             # sequences per step
    N: int = 256           # tokens per sequence
    d: int = 64            # model and head width
    rank: int = 4          # rank of the token inputs' structure
    gain: float = 12.0     # size of the sink key input
    lr: float = 0.05
    steps: int = 300
    seed: int = 2024
    power_iters: int = 4   # power-iteration steps per spectral norm per training step


def spectral_norm(W, v, iters: int):
    """Largest singular value of W by power iteration on W^T W, starting
    from v (a unit vector, updated in place is not assumed: the new vector
    is returned).  Returns (sigma, v)."""
    for _ in range(iters):
        u = W @ v
        v = W.transpose(-1, -2) @ u
        v = v / v.norm()
    return float((W @ v).norm()), v


class Toy:
    """Data, weights and the gradient computations of the toy layer (GPU)."""

    def __init__(self, cfg: ToyConfig, tied: bool):
        import numpy as np
        import torch
        self.cfg, self.tied, self.torch = cfg, tied, torch
        rng = np.random.default_rng([cfg.seed, 0xB1A5])
        cuda = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()  # noqa: E731
        d, r = cfg.d, cfg.rank
        self.basis = cuda(rng.standard_normal((r, d)) / math.sqrt(r))
        self.common = cuda(rng.standard_normal(d))
        self.W0 = [cuda(rng.standard_normal((d, d)) / math.sqrt(d)) for _ in range(3)]
        self.teacher = cuda(rng.standard_normal((d, d)) / math.sqrt(d))
        sink = cuda(rng.standard_normal(d))
        sink = sink / sink.norm() * math.sqrt(d)
        if float((self.common @ self.W0[0]) @ (sink @ self.W0[1])) < 0:  # queries favour the sinks
            sink = -sink
        self.sink = cfg.gain * sink
        self.sink2 = self.sink if tied else self.sink + 0.01 * cfg.gain * cuda(rng.standard_normal(d))
        self.scale = 1.0 / math.sqrt(d)

    def batch(self, t: int):
        """Token inputs X, key inputs A (X with the two sinks), targets Y of step t."""
        torch, cfg = self.torch, self.cfg
        g = torch.Generator(device="cuda").manual_seed(7919 * t + 17)
        Z = torch.randn((cfg.B, cfg.N, cfg.rank), generator=g, device="cuda")
        X = self.common + Z @ self.basis + 0.1 * torch.randn((cfg.B, cfg.N, cfg.d), generator=g, device="cuda")
        A = X.clone()
        pos = torch.argsort(torch.rand((cfg.B, cfg.N), generator=g, device="cuda"), dim=1)[:, :2]
        rows = torch.arange(cfg.B, device="cuda")
        A[rows, pos[:, 0]] = self.sink
        A[rows, pos[:, 1]] = self.sink2
        return X, A, X @ self.teacher

    def qkv_bf16(self, W, X, A):
        """(B, 1, N, d) bf16 q, k, v: the layer's projections rounded once."""
        torch = self.torch
        return [(x @ w).to(torch.bfloat16).unsqueeze(1).contiguous() for x, w in zip((X, A, X), W)]

    def attention_grads(self, W, X, A, Y, stabilize: bool):
        """Attention forward and backward through the library: returns the
        bf16 q, k, v, dO, the outputs (O, LSE, dq, dk, dv) and the weight
        gradients they give."""
        import precision_numerics_fa_amd as fa
        torch = self.torch
        q, k, v = self.qkv_bf16(W, X, A)
        o, lse = fa.fwd(q, k, v, causal=False, scale=self.scale, stabilize=stabilize)
        do = ((2.0 / Y.numel()) * (o.float().squeeze(1) - Y)).to(torch.bfloat16).unsqueeze(1).contiguous()
        dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=False, scale=self.scale)
        gW = [(x.transpose(-1, -2) @ g.float().squeeze(1)).sum(0) for x, g in zip((X, A, X), (dq, dk, dv))]
        return {"q": q, "k": k, "v": v, "do": do, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "gW": gW}

    def reference_grads(self, W, X, A, Y):
        """float32 weight gradients of the same loss on the same bf16 q, k, v
        (the rounding of q, k, v passed straight through), the loss, the
        fraction of rows with a repeated maximum and the top-2 attention mass."""
        torch = self.torch
        Wt = [w.clone().requires_grad_(True) for w in W]
        q, k, v = [(t.to(torch.bfloat16).float() - t).detach() + t for t in (X @ Wt[0], A @ Wt[1], X @ Wt[2])]
        s = (q @ k.transpose(-1, -2).contiguous()) * self.scale
        p = torch.softmax(s, dim=-1)
        loss = ((p @ v - Y) ** 2).mean()
        loss.backward()
        s, p = s.detach(), p.detach()
        tied = float(((s == s.max(dim=-1, keepdim=True).values).sum(-1) >= 2).float().mean())
        top2 = float(p.topk(2, dim=-1).values.sum(-1).mean())
        return [w.grad for w in Wt], float(loss.detach()), tied, top2


def run(cfg: ToyConfig, tied: bool, record_every: int = 1) -> Dict:
    """One training run of the toy; returns summary statistics and per-step
    curves (every `record_every` steps)."""
    import torch
    toy = Toy(cfg, tied)
    d, T = cfg.d, cfg.steps
    W = {m: [w.clone() for w in toy.W0] for m in ("ref", "off", "on")}
    err_sum = {m: [torch.zeros(d, d, device="cuda") for _ in NAMES] for m in ("off", "on")}
    err_sq = {m: [0.0] * 3 for m in ("off", "on")}
    vec = {}
    unit = torch.ones(d, device="cuda") / math.sqrt(d)
    curves: Dict[str, List] = {"step": []}
    losses, tie_frac, top2, gnorm = [], 0.0, 0.0, [0.0] * 3

    def sigma(key, M):
        # (a cold start converges first; later steps start from the last vector)
        s, vec[key] = spectral_norm(M, vec.get(key, unit), cfg.power_iters if key in vec else 40)
        return s

    for t in range(T):
        X, A, Y = toy.batch(t)
        g_ref, loss, tf, tm = toy.reference_grads(W["ref"], X, A, Y)
        losses.append(loss)
        tie_frac, top2 = tie_frac + tf / T, top2 + tm / T
        gnorm = [a + float(g.norm()) / T for a, g in zip(gnorm, g_ref)]
        for m, stab in (("off", False), ("on", True)):
            g = toy.attention_grads(W["ref"], X, A, Y, stab)["gW"]
            for i in range(3):
                e = g[i] - g_ref[i]
                err_sum[m][i] += e
                err_sq[m][i] += float((e * e).sum())
            W[m] = [w - cfg.lr * gi for w, gi in zip(W[m], toy.attention_grads(W[m], X, A, Y, stab)["gW"])]
        W["ref"] = [w - cfg.lr * gi for w, gi in zip(W["ref"], g_ref)]
        if t % record_every == 0 or t == T - 1:
            curves["step"].append(t + 1)
            for m in ("ref", "off", "on"):
                for i, name in enumerate(NAMES[:2]):
                    curves.setdefault(f"sigma_{name}_{m}", []).append(sigma((m, name), W[m][i]))
            for m in ("off", "on"):
                for i, name in enumerate(NAMES[:2]):
                    curves.setdefault(f"sigma_accumulated_error_{name}_{m}", []).append(
                        sigma(("err", m, name), err_sum[m][i]))
    torch.cuda.synchronize()
    res = {"tied_row_fraction": round(tie_frac, 4), "top2_attention_mass": round(top2, 3),
           "loss_first": round(losses[0], 5), "loss_last": round(losses[-1], 5),
           "mean_ref_grad_norm": {n: float(f"{g:.3e}") for n, g in zip(NAMES, gnorm)}}
    for m in ("off", "on"):
        for i, name in enumerate(NAMES):
            S = err_sum[m][i]
            res[f"{name}_fix_{m}"] = {
                "accumulation_ratio": round(float(S.norm()) / max(math.sqrt(err_sq[m][i]), 1e-30), 2),
                "rms_error_per_step": float(f"{math.sqrt(err_sq[m][i] / T):.3e}"),
                "accumulated_error": float(f"{float(S.norm()):.3e}")}
    for m in ("off", "on"):
        res[f"weight_distance_from_ref_{m}"] = float(
            f"{math.sqrt(sum(float(((a - b) ** 2).sum()) for a, b in zip(W[m], W['ref']))):.3e}")
    res["curves"] = {k: [round(x, 6) if isinstance(x, float) else x for x in v] for k, v in curves.items()}
    return res


def experiment(cfg: Optional[ToyConfig] = None, record_every: int = 1) -> Dict:
    cfg = cfg or ToyConfig()
    return {"config": dataclasses.asdict(cfg), "independent_errors_ratio": 1.0,
            "one_direction_ratio": round(math.sqrt(cfg.steps), 2),
            "tied": run(cfg, True, record_every), "untied_control": run(cfg, False, record_every)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--steps", type=int, default=ToyConfig.steps)
    ap.add_argument("--record-every", type=int, default=1)
    ap.add_argument("--out", default=None, help="write the full record (with curves) as JSON here")
    a = ap.parse_args(argv)
    out = experiment(ToyConfig(steps=a.steps), a.record_every)
    if a.out:
        with open(a.out, "w") as f:
            json.dump(out, f)
    brief = {k: ({kk: vv for kk, vv in v.items() if kk != "curves"} if isinstance(v, dict) else v)
             for k, v in out.items()}
    print(json.dumps({"bias_toy": brief}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
