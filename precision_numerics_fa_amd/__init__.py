"""Tiled BF16 (and FP16) FlashAttention forward/backward for AMD MI355X (gfx950).

Thin Python binding of the C ABI in include/fa.h (libfa.so, built in-tree by
``python -m precision_numerics_fa_amd.build``).  PyTorch supplies device
memory and the current stream; every step of the computation runs in the HIP
kernels.  There is no fallback: if the library is missing or the device is
not a gfx950 GPU, the calls raise.

    o, lse = fwd(q, k, v, causal=True, stabilize=True)
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal=True)
    o = attention(q, k, v, causal=True, stabilize=True)   # differentiable (autograd)

Tensors are torch.bfloat16, shape (B, H, N, d), contiguous, on the current
CUDA (HIP) device; LSE is float32 (B, H, N).  fwd_ex / bwd_ex take
torch.float16 tensors as well (the element type follows q).

    o, lse = base_fwd(q, k, v, causal=True)   # unfused FP32-accumulating baseline

base_fwd is the baseline attention the FlashAttention kernels are compared
with (S and P materialised in HBM, softmax over whole rows in FP32); its three
steps are also exposed (base_scores, base_softmax, base_pv).
"""
from ._lib import (  # noqa: F401
    FA_BF16,
    FA_F16,
    FAError,
    attention,
    base_fwd,
    base_ld,
    base_pv,
    base_scores,
    base_softmax,
    base_workspace_bytes,
    bwd,
    bwd_ex,
    bwd_grads,
    bwd_dkdv,
    bwd_dot,
    bwd_noalloc,
    NOALLOC_MAX_ROWS,
    bwd_dq,
    fwd,
    fwd_diag,
    fwd_ex,
    fwd_split,
    fwd_split_workspace_bytes,
    fwd_tile,
    lib_path,
    hbm_probe,
    issue_probe,
    ISSUE_PROBE_KINDS,
    load,
    mfma_probe,
    stabilize_params,
    status_string,
    version,
    workspace_bytes,
)
