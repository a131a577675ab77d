"""Build the HIP library libfa.so in-tree for gfx950 (MI355X).

    python -m precision_numerics_fa_amd.build [--verbose]

One hipcc invocation compiles the kernels and the C ABI into
precision_numerics_fa_amd/libfa.so.  Packed FP32 VALU instructions are
disabled for all device code (-packed-fp32-ops).  Floating-point contraction
is off: a multiply-add is fused only where the source calls fmaf, so every
rounding site is the one written in the kernel (and the stabilised and plain
kernel instances round identically on rows the shift never touches).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-shared", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=off",
            "-Wall", "-Wno-unused-function",
            "-I", INCLUDE, "-I", CSRC, *extra,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    # a kernel whose host-side launch stub was not emitted would only fail
    # when the library is loaded; refuse such a build here
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        missing = [ln.split()[-1] for ln in und.splitlines() if "__device_stub__" in ln]
        if missing:
            os.remove(tmp)
            raise RuntimeError("hipcc produced a library with undefined kernel stubs: " + ", ".join(missing[:4]))
    os.replace(tmp, LIB)
    if verbose:
        print(" ".join(cmd))
        for ln in msgs:
            print(ln)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
