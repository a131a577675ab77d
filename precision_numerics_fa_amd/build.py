"""Build the HIP library libfa.so in-tree for gfx950 (MI355X).

    python -m precision_numerics_fa_amd.build [--verbose]

Each source is compiled to an object by hipcc (in parallel), and the objects
are linked into precision_numerics_fa_amd/libfa.so.  Packed FP32 VALU
instructions are disabled for all device code (-packed-fp32-ops).
Floating-point contraction is off: a multiply-add is fused only where the
source calls fmaf, so every rounding site is the one written in the kernel
(and the stabilised and plain kernel instances round identically on rows the
shift never touches).  The inline-assembly HBM->LDS copies name M0 as clobbered
(-Wno-inline-asm silences the note that M0 is a reserved register: the
compiler keeps no value of its own in M0 across them).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_base.hip", "fa_probe.hip", "fa_api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=off", "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
          "-Rpass-analysis=kernel-resource-usage"]
PER_SOURCE = {}
NOISE = "is not a recognized feature for this target"


def compile_commands(objdir: str) -> list:
    return [[hipcc(), *COMMON, "-I", INCLUDE, "-I", CSRC, *PER_SOURCE.get(src, []),
             "-c", os.path.join(CSRC, src), "-o", os.path.join(objdir, src + ".o")] for src in SOURCES]


def link_command(objdir: str, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
            *[os.path.join(objdir, s + ".o") for s in SOURCES], "-o", out]


def _run(cmds: list) -> list:
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True) for c in cmds]
    msgs = []
    for cmd, p in zip(cmds, procs):
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if NOISE not in ln and ln.strip()]
        if p.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
        msgs += lines
    return msgs


RESOURCE = re.compile(r"remark: +(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]): (\S+)")


def kernel_resources(msgs: list) -> dict:
    """Per-kernel registers, scratch and occupancy from the compiler's
    kernel-resource-usage remarks."""
    table, cur = {}, None
    for ln in msgs:
        m = RESOURCE.search(ln)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = table.setdefault(val, {})
        elif cur is not None:
            cur[key.split()[0]] = int(val)
    return table


def check_resources(table: dict) -> None:
    """Refuse kernels that spill.  The tile copies are inline-asm loads the
    compiler does not count; a spill reload inside a loop gets a partial
    vmcnt wait computed without them, which is not a wait for the reload."""
    spills = [k for k, v in table.items() if v.get("ScratchSize", 0) > 0]
    if spills:
        raise RuntimeError("kernels use scratch (register spills): " + ", ".join(spills))


def build(verbose: bool = False, out: str = LIB) -> str:
    tmp = out + ".tmp"
    objdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        cmds = compile_commands(objdir)
        msgs = _run(cmds)
        resources = kernel_resources(msgs)
        msgs = [ln for ln in msgs if "kernel-resource-usage" not in ln]
        check_resources(resources)
        link = link_command(objdir, tmp)
        msgs += _run([link])
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    # a kernel whose host-side launch stub was not emitted would only fail
    # when the library is loaded; refuse such a build here
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        missing = [ln.split()[-1] for ln in und.splitlines() if "__device_stub__" in ln]
        if missing:
            os.remove(tmp)
            raise RuntimeError("hipcc produced a library with undefined kernel stubs: " + ", ".join(missing[:4]))
    os.replace(tmp, out)
    if verbose:
        for c in cmds + [link]:
            print(" ".join(c))
        for ln in msgs:
            print(ln)
        for name, v in sorted(resources.items()):
            print(f"{name}: {v}")
    return out


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    print(build(verbose="--verbose" in sys.argv, out=os.path.abspath(args[0]) if args else LIB))
