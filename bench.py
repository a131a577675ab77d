"""Benchmark of the tiled BF16 attention hot path on one MI355X.

One step = one full pass of the hot path on the Llama-2-7B attention shape
(B=4, H=32, N=4096, d=128, causal, stabilised shift on): fa_fwd, then the
backward's two launches (row-dot prepass, then dQ/dK/dV in one launch).  Inputs
are resident in HBM before the timed region.  The step is timed as a whole
(synchronised wall clock) and each kernel with HIP events on the stream it is
launched on.  Outside the timed step, the same inputs also go through the
unfused FP32-accumulating baseline attention (fa_base_*: its three kernels
timed against the HBM roofline), and FlashAttention (fix on and off) and the
baseline are compared with the float64 oracle on the same heads (page 3's
deviation comparison).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
    python bench.py --sweep [--steps 20]      # per-workload forward/backward table

Prints one JSON line.  FLOP are algorithmic: forward 4*B*H*N^2*d halved for
causal; backward 2.5x the forward (five N^2 d products against two).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
METRIC = "attn fwd/bwd TFLOP/s & % BF16 MFMA peak (1 GPU); max/mean |err| vs FP64 oracle"
KERNEL_SOURCES = ["fa_device.hpp", "fa_fwd.hip", "fa_bwd.hip"]
BASE_KERNEL_SOURCES = ["fa_device.hpp", "fa_base.hip"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--issue-probe", action="store_true",
                    help="print the instruction-issue probe's table (fa_issue_probe) and exit")
    ap.add_argument("--power", action="store_true",
                    help="print the board power and graphics clock (amd-smi, sampled midway through "
                         "a few seconds of back-to-back calls) for the c4 forward and backward and for "
                         "the probe's MFMA, LDS-read and VALU kinds, one JSON line each, and exit")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the short timing of the other bf16 workloads after the step")
    ap.add_argument("--cpu-heads", type=int, default=128,
                    help="heads the CPU oracle checks and times (all 128 of the workload by default)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step benchmark, time the forward (fix on and off) and the "
                         "backward on every workload c1..c5 and print one JSON line per workload")
    ap.add_argument("--bias-toy", action="store_true",
                    help="instead of the step benchmark, measure how the attention gradient's "
                         "rounding error accumulates over training steps of a toy attention layer "
                         "with repeated tokens, fix off and on (one JSON line)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times "
                         "(calibrates the HBM byte counters) and exit")
    return ap.parse_args()


def copy_probe(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}), flush=True)


def source_digest(sources=None) -> str:
    """Digest of the kernel sources with comments and blank space removed, so
    that the stored counter figures stay valid across comment-only edits."""
    h = hashlib.sha256()
    for s in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "precision_numerics_fa_amd", "csrc", s)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _counter_record(name: str, kernel: str):
    """Per-kernel record of a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None.  The baseline's kernels
    carry the digest of their own sources."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if kernel.startswith("base_"):
        if rec.get("base_source_digest") != source_digest(BASE_KERNEL_SOURCES):
            return None
        return rec.get("base_kernels", {}).get(kernel)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("kernels", {}).get(kernel)


def counter_traffic(kernel: str):
    """HBM bytes per launch for `kernel` (FETCH_SIZE + WRITE_SIZE, calibrated)."""
    k = _counter_record("hbm_traffic.json", kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def counter_mfma_busy(kernel: str):
    """Fraction of the kernel's cycles the MFMA pipes were busy (SQ counters,
    every MFMA counted, recomputation included; independent of the clock)."""
    k = _counter_record("sq_counters.json", kernel)
    return None if k is None else k.get("mfma_pipe_busy")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path needs no collectives; "
              f"heads shard across GPUs with no communication). --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fa_inputs as F
    import precision_numerics_fa_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    fa.load()
    if args.sweep:
        sweep(args)
        return
    if args.issue_probe:
        issue_probe_table()
        return
    if args.power:
        power_table()
        return
    if args.bias_toy:
        bias_toy(args)
        return

    w = F.WORKLOADS["c4"].with_shape(with_do=True)
    B, H, N, d = w.B, w.H, w.N, w.d
    t0 = time.time()
    full = F.full(w)
    gen_s = time.time() - t0
    dev = {n: torch.from_numpy(full[n].view(np.int16)).view(torch.bfloat16).cuda()
           for n in ("q", "k", "v", "do")}
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dvec = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stab = True

    # one step = fa_fwd, then fa_bwd's two launches (row-dot, then dQ/dK/dV
    # in one launch), with events between the launches
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fwd(q, k, v, causal=True, stabilize=stab, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        fa.bwd_dot(o, do, dvec)
        if ev is not None:
            ev[2].record()
        fa.bwd_grads(q, k, v, do, lse, dvec, causal=True, dq=dq, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps
    names = ["fwd", "bwd_dot", "bwd_grads"]
    kern_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events])) for i, n in enumerate(names)}

    # the cost of the fix: the forward alone, fix on and off interleaved in
    # rounds of the same length on the same inputs (so that clock and
    # thermal drift fall on both alike)
    rounds = {True: [], False: []}
    reps = max(5, args.steps // 2)
    for r in range(6):
        for flag in (True, False):
            for _ in range(2):
                fa.fwd(q, k, v, causal=True, stabilize=flag, out=o, lse=lse)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fa.fwd(q, k, v, causal=True, stabilize=flag, out=o, lse=lse)
            e1.record()
            torch.cuda.synchronize()
            rounds[flag].append(e0.elapsed_time(e1) / reps)
    fwd_ab = {("on" if flag else "off"): {"min_ms": round(min(ts), 4),
                                         "median_ms": round(float(np.median(ts)), 4)}
              for flag, ts in rounds.items()}
    fwd_ab["cost_of_fix_pct"] = round(100 * (np.median(rounds[True]) / np.median(rounds[False]) - 1), 2)
    fwd_ab["rounds"] = f"6 interleaved rounds of {reps} calls each"
    fwd_off_ms = float(np.median(rounds[False]))
    fa.fwd(q, k, v, causal=True, stabilize=stab, out=o, lse=lse)  # restore the stabilised outputs
    fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()

    fwd_flop = 4.0 * B * H * N * N * d / 2.0
    bwd_flop = 2.5 * fwd_flop
    step_flop = fwd_flop + bwd_flop
    value = step_flop / (ms_step * 1e-3) / 1e12
    # algorithmic FLOP attributed to each kernel: the dQ/dK/dV launch carries
    # the backward's five products (its recomputed S and dP are not counted)
    kflop = {"fwd": fwd_flop, "bwd_dot": 0.0, "bwd_grads": bwd_flop}
    elem = B * H * N * d
    kbytes = {"fwd": 4 * elem * 2 + B * H * N * 4, "bwd_dot": 2 * elem * 2 + B * H * N * 4,
              "bwd_grads": 7 * elem * 2 + 2 * B * H * N * 4}
    kernel_names = {"fwd": "fwd_kernel", "bwd_dot": "bwd_dot_kernel", "bwd_grads": "bwd_grads_kernel"}
    kernels = {}
    for n in names:
        t = kern_ms[n] * 1e-3
        if kflop[n] > 0:
            ach = kflop[n] / t / 1e12
            kernels[n] = {"ms": round(kern_ms[n], 4), "bound": "mfma", "achieved": round(ach, 1),
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = kbytes[n] / t / 1e9
            kernels[n] = {"ms": round(kern_ms[n], 4), "bound": "hbm", "achieved": round(ach, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
        kernels[n]["traffic"] = counter_traffic(kernel_names[n])
        if kflop[n] > 0:
            kernels[n]["mfma_pipe_busy"] = counter_mfma_busy(kernel_names[n])
    peaks = measured_peaks()
    for n in names:
        meas = peaks["mfma_bf16_tflops"] if kernels[n]["bound"] == "mfma" else peaks["hbm_read_gbs"]
        kernels[n]["frac_of_measured"] = round(kernels[n]["achieved"] / meas, 4)
    dominant = max(names, key=lambda n: kern_ms[n])
    roofline = dict(kernels[dominant])
    roofline.pop("ms")
    roofline["kernel"] = kernel_names[dominant]

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama2-7b attention fwd+bwd, causal, stabilized (B=4 H=32 N=4096 d=128)",
                   "B": B, "H": H, "N": N, "d": d, "causal": True, "stabilize": stab,
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flop / (kern_ms["fwd"] * 1e-3) / 1e12, 1),
        "fwd_pct_peak": round(100 * fwd_flop / (kern_ms["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "bwd_tflops": round(bwd_flop / (sum(kern_ms[n] for n in names[1:]) * 1e-3) / 1e12, 1),
        "fwd_stabilize_off_ms": round(fwd_off_ms, 4),
        "fwd_stabilize_on_ms": round(float(np.median(rounds[True])), 4),
        "fwd_fix_on_off_interleaved": fwd_ab,
        "kernels": kernels,
        "roofline": roofline,
        "measured_peaks": peaks,
        "input_gen_s": round(gen_s, 2),
    }

    out["f16"] = f16_leg(args, fwd_flop, bwd_flop)
    o_plain = torch.empty_like(q)
    fa.fwd(q, k, v, causal=True, stabilize=False, out=o_plain, lse=torch.empty_like(lse))
    base = baseline_leg(args, q, k, v, fwd_flop, kern_ms["fwd"])
    out["baseline_fp32acc"] = base.pop("record")
    if not args.no_other_workloads:
        out["other_workloads"] = other_workloads_leg()
    if not args.no_cpu_baseline:
        out["tie_bias"] = tie_bias_leg()
        out.update(cpu_baseline_leg(w, full, o, lse, dq, dk, dv, args.cpu_heads, fwd_flop + bwd_flop,
                                    compare={"flash_fix_on": o, "flash_fix_off": o_plain,
                                             "baseline_fp32acc": base["o"]}))
    print(json.dumps(out), flush=True)


def tie_bias_leg(batches=(0, 1, 2, 3)):
    """The mean signed error on rows whose maximum repeats, with the fix off
    and on: the tie-heavy workload (8, 12, 1024, 64, causal, Q and K x 4, 5%
    of rows given a repeated maximum), FlashAttention on the GPU against the
    float64 oracle on the heads of the given batch entries.  "aligned" signs
    each error by the side of the tied values' mean the exact output lies on
    (the direction of the bias); non-tie rows are the control."""
    import numpy as np
    import torch

    import fa_inputs as F
    import precision_numerics_fa_amd as fa
    from oracle import metrics as Mt
    from oracle import reference as REF

    w = F.WORKLOADS["c2"]
    full = F.full(w)
    q, k, v = (torch.from_numpy(full[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v"))
    outs = {flag: fa.fwd(q, k, v, causal=True, stabilize=flag)[0].float().cpu().numpy() for flag in (False, True)}
    rec = {"workload": f"{w.B}x{w.H}x{w.N}x{w.d} causal, Q and K x 4, 5% repeated-maximum rows",
           "heads": len(batches) * w.H}
    diffs = {False: [], True: []}
    refs, metas = [], []
    for b in batches:
        qh, kh, vh = (F.bf16_bits_to_f32(full[n][b]).astype(np.float64) for n in ("q", "k", "v"))
        o_ref, _ = REF.forward(qh, kh, vh, w.scale, True)
        refs.append(o_ref)
        metas.append(REF.tie_metadata(qh, kh, vh, w.scale, True))
    o_ref = np.stack(refs)
    count = np.stack([m["count"] for m in metas])
    tmean = np.stack([m["tie_mean"] for m in metas])
    for flag in (False, True):
        o = outs[flag][list(batches)]
        rep = Mt.tie_report(o, o_ref, count, tmean)
        rec["fix_on" if flag else "fix_off"] = {
            part: {key: (round(val, 9) if isinstance(val, float) else val) for key, val in stats.items()}
            for part, stats in rep.items()}
    del q, k, v
    torch.cuda.empty_cache()
    return rec


def measured_peaks():
    """The ceilings this chip sustains, measured in the same run: dense bf16
    MFMA throughput from the library's probe kernel (register operands only),
    and HBM read bandwidth from its read probe over 2 GiB.
    Each is the best of five timed launches."""
    import torch

    import precision_numerics_fa_amd as fa

    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    flop, _ = fa.mfma_probe(2048, 2000, out=out)
    fa.mfma_probe(2048, 2000, out=out)
    t_mfma = min(_timed(lambda: fa.mfma_probe(2048, 2000, out=out), 1) for _ in range(5))
    src = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    sink = fa.hbm_probe(src)
    t_read = min(_timed(lambda: fa.hbm_probe(src, sink), 1) for _ in range(5))
    nbytes = src.numel() * 4
    del src, sink, out
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(flop / (t_mfma * 1e-3) / 1e12, 1),
            "hbm_read_gbs": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "how": "fa_mfma_probe: bf16 MFMA-only kernel (2048 workgroups, 8 chains per wave); fa_hbm_probe: "
                   "2 GiB read with 16-byte loads; best of 5 each"}


def baseline_leg(args, q, k, v, fwd_flop, fa_fwd_ms):
    """The unfused FP32-accumulating baseline on the same inputs: each of its
    three launches timed with HIP events, against the HBM roofline with the
    bytes the algorithm must move (Q, K in and the visible scores out; the
    scores in and the probabilities out; the probabilities and V in and O
    out).  Returns the record and the baseline's O for the deviation study."""
    import torch

    import precision_numerics_fa_amd as fa

    B, H, N, d = (int(x) for x in q.shape)
    ld = fa.base_ld(N)
    S = torch.empty((B, H, N, ld), dtype=torch.float32, device="cuda")
    P = torch.empty((B, H, N, ld), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty_like(q)
    lb = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    steps = [("scores", lambda: fa.base_scores(q, k, causal=True, s=S)),
             ("softmax", lambda: fa.base_softmax(S, causal=True, p=P, lse=lb)),
             ("pv", lambda: fa.base_pv(P, v, causal=True, out=ob))]
    reps = max(3, args.steps // 5)
    for _ in range(2):
        for _, fn in steps:
            fn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        for i, (_, fn) in enumerate(steps):
            ev[r][i].record()
            fn()
        ev[r][3].record()
    torch.cuda.synchronize()
    ms = {n: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / reps for i, (n, _) in enumerate(steps)}
    vis = B * H * N * (N + 1) // 2          # causal scores
    elem = B * H * N * d
    algo = {"scores": 2 * elem * 2 + vis * 4, "softmax": vis * 4 + vis * 2 + B * H * N * 4,
            "pv": vis * 2 + elem * 2 + elem * 2}
    names = {"scores": "base_scores_kernel", "softmax": "base_softmax_kernel", "pv": "base_pv_kernel"}
    kernels = {}
    for n in ms:
        ach = algo[n] / (ms[n] * 1e-3) / 1e9
        kernels[n] = {"kernel": names[n], "ms": round(ms[n], 4), "bound": "hbm", "achieved": round(ach, 1),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                      "bytes": algo[n], "traffic": counter_traffic(names[n])}
    total = sum(ms.values())
    # the same call through the one-shot entry point, bitwise the steps' result
    ob2, _ = fa.base_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    same = bool(torch.equal(ob, ob2))
    del S, P, ob2
    torch.cuda.empty_cache()
    rec = {"workload": f"same inputs (B={B} H={H} N={N} d={d}, causal): unfused baseline attention with FP32 "
                       "accumulation, S (fp32) and P (bf16) materialised in HBM",
           "ms": round(total, 4), "tflops": round(fwd_flop / (total * 1e-3) / 1e12, 1),
           "flash_fwd_speedup": round(total / fa_fwd_ms, 2), "kernels": kernels,
           "one_shot_equals_steps": same}
    return {"record": rec, "o": ob}


def f16_leg(args, fwd_flop, bwd_flop):
    """The same shape in IEEE binary16 (fa_fwd_ex / fa_bwd_ex): forward with
    the fix on, and the whole backward, each timed alone with HIP events."""
    import numpy as np
    import torch

    import fa_inputs as F
    import precision_numerics_fa_amd as fa

    w = F.WORKLOADS["c4h"].with_shape(with_do=True)
    full = F.full(w)
    q, k, v, do = (torch.from_numpy(full[n].view(np.int16)).view(torch.float16).cuda()
                   for n in ("q", "k", "v", "do"))
    del full
    res = {}
    fwd = lambda: res.update(zip("ol", fa.fwd_ex(q, k, v, causal=True, stabilize=True)))
    t_fwd = _timed(fwd, args.steps)
    fwd()
    t_bwd = _timed(lambda: fa.bwd_ex(q, k, v, res["o"], do, res["l"], causal=True), args.steps)
    del q, k, v, do, res
    torch.cuda.empty_cache()
    return {"workload": "same shape, IEEE binary16 inputs and rounding sites",
            "fwd_ms": round(t_fwd, 4), "fwd_tflops": round(fwd_flop / (t_fwd * 1e-3) / 1e12, 1),
            "fwd_pct_peak": round(100 * fwd_flop / (t_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "bwd_ms": round(t_bwd, 4), "bwd_tflops": round(bwd_flop / (t_bwd * 1e-3) / 1e12, 1)}


def _timed(fn, reps):
    import torch
    for _ in range(max(2, reps // 5)):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def issue_probe_table(blocks: int = 1024, iters: int = 2048):
    """fa_issue_probe for every kind at one and two waves per SIMD: the time
    of one loop iteration of a SIMD's waves (the fastest of three launches)."""
    import torch

    import precision_numerics_fa_amd as fa

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    rows = []
    for kind, name in enumerate(fa.ISSUE_PROBE_KINDS):
        rec = {"kind": kind, "work_per_wave_and_iteration": name}
        for w in (1, 2):
            if kind == 7 and w == 1:
                continue
            fn = lambda: fa.issue_probe(kind, w, blocks, iters, out)  # noqa: E731
            fn()
            best = min(_timed(fn, 1) for _ in range(3))
            rec[f"ns_per_iteration_{w}_wave" + ("s" if w == 2 else "")] = round(
                best * 1e6 / (blocks / cus) / iters, 2)
        rows.append(rec)
        print(json.dumps(rec), flush=True)
    return rows


def _smi_sample():
    """Board power (W) and the mean graphics clock (MHz) over the XCDs from
    `amd-smi metric --power --clock`, or None where the tool gives none."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock"], capture_output=True, text=True,
                           timeout=60)
    except (OSError, subprocess.TimeoutExpired):
        return None, None
    p = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
    clk = [float(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", r.stdout)]
    return (float(p.group(1)) if p else None), (round(sum(clk) / len(clk), 1) if clk else None)


def power_table(seconds: float = 6.0):
    """What each kind of work draws: calls queued back to back for `seconds`,
    power and clock sampled halfway, then the rate from HIP events."""
    import torch

    import fa_inputs as F
    import precision_numerics_fa_amd as fa

    w = F.WORKLOADS["c4"].with_shape(with_do=True)
    B, H, N, d = w.B, w.H, w.N, w.d
    g = torch.Generator(device="cuda").manual_seed(0)
    q, k, v, do = (torch.randn(B, H, N, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(4))
    scale = d ** -0.5
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale, stabilize=True)
    flop_f = 4.0 * B * H * N * N * d / 2
    blocks, iters = 1024, 4096
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    cases = [
        ("c4 forward, fix on", lambda: fa.fwd(q, k, v, causal=True, scale=scale, stabilize=True),
         lambda ms: {"tflops": round(flop_f / ms / 1e9, 1)}),
        ("c4 backward", lambda: fa.bwd(q, k, v, o, do, lse, causal=True, scale=scale),
         lambda ms: {"tflops": round(2.5 * flop_f / ms / 1e9, 1)}),
    ]
    probe_rate = {
        0: lambda ms: {"tflops": round(blocks * 8 * iters * 8 * 32768 / ms / 1e9, 1)},
        9: lambda ms: {"tflops": round(blocks * 8 * iters * 8 * 32768 / ms / 1e9, 1),
                       "lds_bytes_per_clk_per_cu_at_2400mhz": round(
                           blocks * 8 * iters * 8 * 1024 / (ms * 1e-3) / cus / 2.4e9, 1)},
        8: lambda ms: {"lds_bytes_per_clk_per_cu_at_2400mhz": round(
            blocks * 8 * iters * 8 * 1024 / (ms * 1e-3) / cus / 2.4e9, 1)},
        10: lambda ms: {"lds_bytes_per_clk_per_cu_at_2400mhz": round(
            blocks * 8 * iters * 16 * 512 / (ms * 1e-3) / cus / 2.4e9, 1)},
        11: lambda ms: {"tflops": round(blocks * 8 * iters * 8 * 32768 / ms / 1e9, 1),
                        "lds_bytes_per_clk_per_cu_at_2400mhz": round(
                            blocks * 8 * iters * 8 * 1024 / (ms * 1e-3) / cus / 2.4e9, 1)},
        1: lambda ms: {"ns_per_iteration": round(ms * 1e6 / (blocks / cus) / iters, 1)},
        4: lambda ms: {"ns_per_iteration": round(ms * 1e6 / (blocks / cus) / iters, 1)},
    }
    for kind in (0, 8, 9, 10, 11, 1, 4):
        cases.append((f"probe: {fa.ISSUE_PROBE_KINDS[kind]}, two waves per SIMD",
                      (lambda kk: lambda: fa.issue_probe(kk, 2, blocks, iters, out))(kind), probe_rate[kind]))
    rows = []
    for name, fn, rate in cases:
        ms = min(_timed(fn, 3) for _ in range(2))
        n = max(1, math.ceil(seconds * 1e3 / ms))
        t0 = time.time()
        for _ in range(n):
            fn()
        while time.time() - t0 < seconds / 2:
            time.sleep(0.05)
        watts, mhz = _smi_sample()
        torch.cuda.synchronize()
        rec = {"power_probe": name, "socket_power_w": watts, "gfx_clock_mhz": mhz, "ms_per_call": round(ms, 4),
               "calls_queued": n}
        rec.update(rate(ms))
        rows.append(rec)
        print(json.dumps(rec), flush=True)
    return rows


def _graph_timed(fn, reps):
    """GPU time of one call of `fn`: `reps` calls captured in one HIP graph,
    the fastest of three replays.  Small launches otherwise measure the
    host's launch rate rather than the kernels."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / reps)
    del g
    return best


def other_workloads_leg(reps: int = 20):
    """The other bf16 workloads' forward (fix on) and backward (row-dot
    pre-pass and dQ/dK/dV launch, outputs preallocated), each as `reps`
    calls captured in a HIP graph and replayed (the fastest of three replays):
    the GPU time per call, without the host's launch overhead, which
    otherwise dominates the small workloads."""
    import numpy as np
    import torch

    import fa_inputs as F
    import precision_numerics_fa_amd as fa

    recs = {}
    for name in ("c1", "c2", "c3", "c5"):
        w = F.WORKLOADS[name].with_shape(with_do=True)
        B, H, N, d = w.B, w.H, w.N, w.d
        full = F.full(w)
        dev = {n: torch.from_numpy(full[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v", "do")}
        del full
        q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        dvec = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        fwd = lambda: fa.fwd(q, k, v, causal=w.causal, stabilize=True, out=o, lse=lse)  # noqa: E731

        def bwd():
            fa.bwd_dot(o, do, dvec)
            fa.bwd_grads(q, k, v, do, lse, dvec, causal=w.causal, dq=dq, dk=dk, dv=dv)
        _timed(fwd, 4 * reps)  # clocks up
        t_fwd = _graph_timed(fwd, reps)
        fwd()
        t_bwd = _graph_timed(bwd, reps)
        pairs = N * (N + 1) / 2 if w.causal else N * N
        fwd_flop = 4.0 * B * H * pairs * d
        recs[name] = {"shape": f"{B}x{H}x{N}x{d}" + (" causal" if w.causal else ""),
                      "fwd_ms": round(t_fwd, 4),
                      "fwd_pct_peak": round(100 * fwd_flop / (t_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                      "bwd_ms": round(t_bwd, 4),
                      "bwd_pct_peak": round(100 * 2.5 * fwd_flop / (t_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        del dev, q, k, v, do, o, lse, dvec, dq, dk, dv
        torch.cuda.empty_cache()
    return recs


def sweep(args):
    """Forward (fix on, fix off) and backward throughput on every workload,
    algorithmic FLOP and bytes as in the step benchmark; for the bf16
    workloads also the split-key forward (2, 4 and 8 key ranges, fix on) and
    the FP32-accumulating baseline.  Every figure is the GPU time of one call:
    `--steps` calls captured in a HIP graph, the fastest of three replays."""
    import numpy as np
    import torch

    import fa_inputs as F
    import precision_numerics_fa_amd as fa

    for name, w0 in F.WORKLOADS.items():
        w = w0.with_shape(with_do=True)
        B, H, N, d = w.B, w.H, w.N, w.d
        full = F.full(w)
        tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
        dev = {n: torch.from_numpy(full[n].view(np.int16)).view(tdt).cuda() for n in ("q", "k", "v", "do")}
        del full
        q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
        reps = args.steps
        res = {}
        if w.dtype == "f16":
            fon = lambda: res.update(zip("ol", fa.fwd_ex(q, k, v, causal=w.causal, stabilize=True)))
            foff = lambda: res.update(zip("ol", fa.fwd_ex(q, k, v, causal=w.causal, stabilize=False)))
            bwd = lambda: fa.bwd_ex(q, k, v, res["o"], do, res["l"], causal=w.causal)
        else:
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
            res.update(o=o, l=lse)
            dvec = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
            grads = [torch.empty_like(q) for _ in range(3)]
            fon = lambda: fa.fwd(q, k, v, causal=w.causal, stabilize=True, out=o, lse=lse)
            foff = lambda: fa.fwd(q, k, v, causal=w.causal, stabilize=False, out=o, lse=lse)

            def bwd():
                fa.bwd_dot(o, do, dvec)
                fa.bwd_grads(q, k, v, do, lse, dvec, causal=w.causal, dq=grads[0], dk=grads[1], dv=grads[2])
        _timed(fon, 4 * reps)  # clocks up
        # fix on and off alternate; each a graph of `reps` calls, fastest replay
        t_on = _graph_timed(fon, reps)
        t_off = _graph_timed(foff, reps)
        t_on = min(t_on, _graph_timed(fon, reps))
        fon()
        t_bwd = _graph_timed(bwd, reps)
        t_split = {}
        if w.dtype == "bf16":
            ws_s = torch.empty(fa.fwd_split_workspace_bytes(B, H, N, d, 8), dtype=torch.uint8, device="cuda")
            o_s = torch.empty_like(q)
            l_s = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
            for ns in (2, 4, 8):
                fn = lambda ns=ns: fa.fwd_split(q, k, v, ns, causal=w.causal, stabilize=True,  # noqa: E731
                                                workspace=ws_s, out=o_s, lse=l_s)
                t_split[ns] = _graph_timed(fn, reps)
            del ws_s, o_s, l_s
        t_base = None
        if w.dtype == "bf16":
            ws = torch.empty(fa.base_workspace_bytes(B, H, N, d, w.causal), dtype=torch.uint8, device="cuda")
            base = lambda: fa.base_fwd(q, k, v, causal=w.causal, workspace=ws)  # noqa: E731
            t_base = _graph_timed(base, reps)
            del ws
        pairs = N * (N + 1) / 2 if w.causal else N * N
        fwd_flop = 4.0 * B * H * pairs * d
        elem = B * H * N * d
        fwd_bytes = 4 * elem * 2 + B * H * N * 4
        rec = {"workload": name, "dtype": w.dtype, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
               "fwd_stab_ms": round(t_on, 4), "fwd_plain_ms": round(t_off, 4),
               "fwd_tflops": round(fwd_flop / (t_on * 1e-3) / 1e12, 1),
               "fwd_pct_peak": round(100 * fwd_flop / (t_on * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
               "fwd_gbs": round(fwd_bytes / (t_on * 1e-3) / 1e9, 1),
               "stabilize_cost_pct": round(100 * (t_on / t_off - 1), 2),
               "bwd_ms": round(t_bwd, 4),
               "bwd_tflops": round(2.5 * fwd_flop / (t_bwd * 1e-3) / 1e12, 1),
               "bwd_pct_peak": round(100 * 2.5 * fwd_flop / (t_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        if t_split:
            best = min(t_split, key=t_split.get)
            rec["fwd_split_ms"] = {str(n_): round(t_, 4) for n_, t_ in t_split.items()}
            rec["fwd_split_best"] = {"splits": best, "ms": round(t_split[best], 4),
                                     "speedup_over_one_pass": round(t_on / t_split[best], 3)}
        if t_base is not None:
            rec["baseline_fp32acc_ms"] = round(t_base, 4)
            rec["flash_speedup_over_baseline"] = round(t_base / t_on, 2)
        print(json.dumps(rec), flush=True)
        del dev, q, k, v, do, res
        torch.cuda.empty_cache()


def cpu_baseline_leg(w, full, o, lse, dq, dk, dv, heads, step_flop, compare=None):
    """Time the float64 oracle on a few heads of the same workload, and check
    the GPU's outputs for those heads against it.  ``compare`` maps names to
    further GPU outputs of the same forward (FlashAttention with the fix on and
    off, the FP32-accumulating baseline), whose deviation from the exact
    result is reported side by side on the same heads (page 3's comparison)."""
    import platform

    import numpy as np
    from threadpoolctl import threadpool_info

    import fa_inputs as F
    from oracle import metrics as Mt
    from oracle import reference as REF

    pairs = F.sample_pairs(w, heads, seed=7)
    f64 = lambda b: F.bf16_bits_to_f32(b).astype(np.float64)  # noqa: E731
    t_cpu = 0.0
    dev_stats = {}
    errs = {"max_abs": 0.0, "mean_abs": [], "max_rel_normwise": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0,
            "lse_max_abs": 0.0}
    for (b, h) in pairs:
        q, k, v, do = (f64(full[n][b, h]) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        o_ref, lse_ref = REF.forward(q, k, v, w.scale, w.causal)
        g_ref = REF.backward(q, k, v, do, w.scale, w.causal)
        t_cpu += time.perf_counter() - t0
        e = Mt.output_errors(o[b, h].float().cpu().numpy(), o_ref)
        errs["max_abs"] = max(errs["max_abs"], e["max_abs"])
        errs["mean_abs"].append(e["mean_abs"])
        errs["max_rel_normwise"] = max(errs["max_rel_normwise"], e["max_rel_normwise"])
        errs["lse_max_abs"] = max(errs["lse_max_abs"], float(np.abs(lse[b, h].cpu().numpy() - lse_ref).max()))
        for n, g, r in (("dq", dq, g_ref[0]), ("dk", dk, g_ref[1]), ("dv", dv, g_ref[2])):
            errs[n] = max(errs[n], Mt.relative_fro(g[b, h].float().cpu().numpy(), r))
        for name, oc in (compare or {}).items():
            ec = Mt.output_errors(oc[b, h].float().cpu().numpy(), o_ref)
            dv_ = dev_stats.setdefault(name, {"max_abs": 0.0, "mean_abs": [], "max_rel_normwise": 0.0,
                                              "max_rel_rowwise": 0.0})
            for key_ in ("max_abs", "max_rel_normwise", "max_rel_rowwise"):
                dv_[key_] = max(dv_[key_], ec[key_])
            dv_["mean_abs"].append(ec["mean_abs"])
    errs["mean_abs"] = float(np.mean(errs["mean_abs"]))
    per_head_flop = step_flop / (w.B * w.H)
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    cpu_tflops = per_head_flop * len(pairs) / t_cpu / 1e12
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            names = [ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")]
        if names:
            cpu_model = names[0]
    except OSError:
        pass
    for dv_ in dev_stats.values():
        dv_["mean_abs"] = float(np.mean(dv_["mean_abs"]))
    # oracle B (the bf16 blocked emulation of the forward) on one of the heads
    from oracle import emulation as EMU
    b0, h0 = pairs[0]
    q0, k0, v0 = (f64(full[n][b0, h0]) for n in ("q", "k", "v"))
    t0 = time.perf_counter()
    EMU.forward(q0, k0, v0, w.scale, w.causal, stabilize=True)
    t_emu = time.perf_counter() - t0
    deviation = None
    if dev_stats:
        deviation = {"heads": len(pairs), "against": "float64 oracle (exact attention)", **dev_stats}
        if "baseline_fp32acc" in dev_stats and "flash_fix_off" in dev_stats:
            b_, f_ = dev_stats["baseline_fp32acc"], dev_stats["flash_fix_off"]
            deviation["flash_over_baseline"] = {
                k_: round(f_[k_] / b_[k_], 3) for k_ in ("max_abs", "mean_abs", "max_rel_normwise",
                                                         "max_rel_rowwise") if b_[k_] > 0}
    return {
        "deviation_study": deviation,
        "cpu_baseline": {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": int(threads),
                         "kind": "oracle",
                         "sample": f"float64 oracle forward+backward on {len(pairs)} of {w.B * w.H} heads "
                                   f"(N={w.N}, d={w.d}, causal), {t_cpu:.1f} s; TFLOP/s under the "
                                   f"GPU's algorithmic FLOP count",
                         "cpu": cpu_model, "host_cpus": os.cpu_count(), "seconds": round(t_cpu, 2),
                         "seconds_per_head": round(t_cpu / len(pairs), 3),
                         "extrapolated_full_s": round(t_cpu / len(pairs) * w.B * w.H, 1),
                         "oracle_b_forward_s_per_head": round(t_emu, 2)},
        "accuracy": {"heads_checked": len(pairs), "o_max_abs": errs["max_abs"], "o_mean_abs": errs["mean_abs"],
                     "o_max_rel_normwise": errs["max_rel_normwise"], "lse_max_abs": errs["lse_max_abs"],
                     "dq_rel": errs["dq"], "dk_rel": errs["dk"], "dv_rel": errs["dv"]},
    }


def bias_toy(args):
    """Bias accumulation in a toy attention layer: precision_numerics_fa_amd.bias_toy."""
    from precision_numerics_fa_amd import bias_toy as toy
    toy.main(["--steps", "300"])


if __name__ == "__main__":
    main()
