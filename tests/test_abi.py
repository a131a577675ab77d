"""The C-ABI library on the host: it loads, exports every function include/fa.h
declares, validates arguments before touching any device, and refuses to run
without a gfx950 GPU (no CPU fallback).  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import precision_numerics_fa_amd as fa
from oracle import emulation as EMU

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p
GOOD = P(4096)  # 16-byte aligned, never dereferenced on these paths


def _declared():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        pytest.fail("libfa.so is not built: run python -m precision_numerics_fa_amd.build")
    return fa.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert isinstance(fa.status_string(code), str) and fa.status_string(code)
    assert fa.status_string(0) == "ok"


def test_stabilize_constants_match_the_oracle(lib):
    dmin, dmax, fold = fa.stabilize_params()
    assert (dmin, dmax, fold) == (EMU.DELTA_MIN, EMU.DELTA_MAX, EMU.FOLD)
    assert fa.stabilize_params(fa.FA_BF16) == EMU.RULES["bf16"]
    assert fa.stabilize_params(fa.FA_F16) == EMU.RULES["f16"]
    x = ctypes.c_float(-7.0)
    assert lib.fa_stabilize_params_ex(5, ctypes.byref(x), None, None) == -2 and x.value == -7.0


def test_workspace_bytes(lib):
    assert fa.workspace_bytes(4, 32, 4096, 128, True) == 4 * 32 * 4096 * 4
    assert fa.workspace_bytes(1, 1, 3, 64, False) == 256
    assert fa.workspace_bytes(1, 1, 0, 64, False) == 0
    assert fa.workspace_bytes(1, 1, 8, 96, False) == 0


def _fwd(lib, q=GOOD, k=GOOD, v=GOOD, o=GOOD, lse=GOOD, B=1, H=1, N=64, d=64, causal=0, scale=0.125,
         stab=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stab, None)


def test_forward_argument_validation(lib):
    assert _fwd(lib, q=None) == -1
    assert _fwd(lib, o=P(4100)) == -1          # misaligned output
    assert _fwd(lib, lse=P(4098)) == -1        # misaligned LSE
    assert _fwd(lib, N=0) == -1
    assert _fwd(lib, B=-1) == -1
    assert _fwd(lib, d=96) == -2
    assert _fwd(lib, d=256) == -2
    assert _fwd(lib, scale=0.0) == -1
    assert _fwd(lib, scale=float("nan")) == -1
    assert _fwd(lib, scale=float("inf")) == -1
    assert _fwd(lib, B=1 << 20, H=1 << 10, N=1 << 12) == -1   # too many elements
    assert lib.fa_fwd_diag(GOOD, GOOD, GOOD, GOOD, GOOD, None, 1, 1, 64, 64, 0, 0.125, 1, None) == -1


def test_backward_argument_validation(lib):
    args = [GOOD] * 9
    need = fa.workspace_bytes(2, 2, 100, 64, True)
    assert lib.fa_bwd(*args, None, need, 2, 2, 100, 64, 1, 0.125, 0, None) == -3
    assert lib.fa_bwd(*args, GOOD, need - 4, 2, 2, 100, 64, 1, 0.125, 0, None) == -3
    assert lib.fa_bwd(None, *args[1:], GOOD, need, 2, 2, 100, 64, 1, 0.125, 0, None) == -1
    assert lib.fa_bwd(*args, GOOD, need, 2, 2, 100, 128 + 1, 1, 0.125, 0, None) == -2
    assert lib.fa_bwd_dot(GOOD, None, GOOD, 1, 1, 8, 64, None) == -1
    assert lib.fa_bwd_dkdv(*[GOOD] * 6, P(4097), GOOD, 1, 1, 8, 64, 1, 0.125, None) == -1
    assert lib.fa_bwd_dq(*[GOOD] * 6, GOOD, 1, 1, 8, 64, 1, -1.0, None) == -1
    assert lib.fa_bwd_grads(*[GOOD] * 6, GOOD, P(4100), GOOD, 1, 1, 8, 64, 1, 0.125, None) == -1
    assert lib.fa_bwd_grads(*[GOOD] * 9, 1, 1, 8, 80, 1, 0.125, None) == -2


def test_noalloc_backward_validation(lib):
    """fa_bwd_noalloc refuses a problem past its fixed scratch, and bad
    arguments, before any device work (here: with no GPU at all)."""
    n = fa.NOALLOC_MAX_ROWS
    assert n == 4194304
    assert lib.fa_bwd_noalloc(*[GOOD] * 9, 1, 1, n + 1, 64, 1, 0.125, 0, None) == -6
    assert lib.fa_bwd_noalloc(*[GOOD] * 9, 2, 4, n // 8 + 1, 64, 1, 0.125, 0, None) == -6
    assert lib.fa_bwd_noalloc(None, *[GOOD] * 8, 1, 1, 8, 64, 1, 0.125, 0, None) == -1
    assert lib.fa_bwd_noalloc(*[GOOD] * 8, P(4098), 1, 1, 8, 64, 1, 0.125, 0, None) == -1
    assert lib.fa_bwd_noalloc(*[GOOD] * 9, 1, 1, 8, 96, 1, 0.125, 0, None) == -2
    assert lib.fa_bwd_noalloc(*[GOOD] * 9, 1, 1, 8, 64, 1, float("nan"), 0, None) == -1
    # a valid call within the limit reaches the device check (no GPU here)
    assert lib.fa_bwd_noalloc(*[GOOD] * 9, 2, 4, n // 8, 64, 1, 0.125, 0, None) == -5


def test_typed_entry_points_validate_dtype_and_arguments(lib):
    """fa_fwd_ex / fa_bwd_ex: an unknown element type is FA_ERR_UNSUPPORTED,
    and both known types go through the same argument checks as fa_fwd/fa_bwd."""
    for bad in (-1, 2, 7):
        assert lib.fa_fwd_ex(bad, GOOD, GOOD, GOOD, GOOD, GOOD, None, 1, 1, 64, 64, 0, 0.125, 0, None) == -2
        need = fa.workspace_bytes(1, 1, 64, 64, False)
        assert lib.fa_bwd_ex(bad, *[GOOD] * 10, need, 1, 1, 64, 64, 0, 0.125, 0, None) == -2
    for dt in (fa.FA_BF16, fa.FA_F16):
        assert lib.fa_fwd_ex(dt, None, GOOD, GOOD, GOOD, GOOD, None, 1, 1, 64, 64, 0, 0.125, 0, None) == -1
        assert lib.fa_fwd_ex(dt, GOOD, GOOD, GOOD, GOOD, GOOD, None, 1, 1, 64, 96, 0, 0.125, 0, None) == -2
        assert lib.fa_fwd_ex(dt, GOOD, GOOD, GOOD, GOOD, GOOD, None, 1, 1, 64, 64, 0, 0.0, 0, None) == -1
        need = fa.workspace_bytes(2, 2, 100, 64, True)
        assert lib.fa_bwd_ex(dt, *[GOOD] * 9, GOOD, need - 4, 2, 2, 100, 64, 1, 0.125, 0, None) == -3
        assert lib.fa_bwd_ex(dt, *[GOOD] * 8, P(4098), GOOD, need, 2, 2, 100, 64, 1, 0.125, 0, None) == -1


def test_no_gpu_means_an_error_not_a_fallback(lib):
    """Valid arguments on a host without a gfx950 GPU: FA_ERR_DEVICE."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _fwd(lib) == -5
    need = fa.workspace_bytes(1, 1, 64, 64, False)
    assert lib.fa_bwd(*[GOOD] * 9, GOOD, need, 1, 1, 64, 64, 0, 0.125, 0, None) == -5
    for dt in (fa.FA_BF16, fa.FA_F16):
        assert lib.fa_fwd_ex(dt, GOOD, GOOD, GOOD, GOOD, GOOD, None, 1, 1, 64, 64, 0, 0.125, 0, None) == -5
        assert lib.fa_bwd_ex(dt, *[GOOD] * 10, need, 1, 1, 64, 64, 0, 0.125, 0, None) == -5
    bneed = fa.base_workspace_bytes(1, 1, 64, 64, False)
    assert lib.fa_base_fwd(*[GOOD] * 6, bneed, 1, 1, 64, 64, 0, 0.125, None) == -5
    assert lib.fa_base_scores(*[GOOD] * 3, 1, 1, 64, 64, 0, 0.125, None) == -5
    assert lib.fa_base_softmax(*[GOOD] * 3, 1, 1, 64, 0, None) == -5
    assert lib.fa_base_pv(*[GOOD] * 3, 1, 1, 64, 64, 0, None) == -5


def test_baseline_sizes_and_validation(lib):
    """fa_base_*: the row stride, the workspace size (S fp32 then P bf16, each
    (B,H,N,ld), P at a 256-byte boundary), the N limit of its softmax, and
    argument checks before any device work."""
    assert [fa.base_ld(n) for n in (1, 63, 64, 65, 4096)] == [64, 64, 64, 128, 4096]
    assert lib.fa_base_ld(0) == 0
    s_bytes = 2 * 3 * 100 * 128 * 4
    assert fa.base_workspace_bytes(2, 3, 100, 64, True) == (s_bytes + 255) // 256 * 256 + 2 * 3 * 100 * 128 * 2
    assert fa.base_workspace_bytes(1, 1, 16384, 64, False) > 0
    assert fa.base_workspace_bytes(1, 1, 16385, 64, False) == 0
    assert fa.base_workspace_bytes(1, 1, 64, 96, False) == 0
    need = fa.base_workspace_bytes(1, 1, 64, 64, False)
    base = lambda *a: lib.fa_base_fwd(*a)  # noqa: E731
    assert base(GOOD, GOOD, GOOD, GOOD, GOOD, None, need, 1, 1, 64, 64, 0, 0.125, None) == -3
    assert base(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need - 1, 1, 1, 64, 64, 0, 0.125, None) == -3
    assert base(GOOD, GOOD, GOOD, GOOD, GOOD, P(4096 + 16), need, 1, 1, 64, 64, 0, 0.125, None) == -3
    assert base(None, GOOD, GOOD, GOOD, GOOD, GOOD, need, 1, 1, 64, 64, 0, 0.125, None) == -1
    assert base(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need, 1, 1, 20000, 64, 0, 0.125, None) == -2
    assert base(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need, 1, 1, 64, 80, 0, 0.125, None) == -2
    assert base(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need, 1, 1, 64, 64, 0, 0.0, None) == -1
    assert lib.fa_base_scores(GOOD, GOOD, P(4100), 1, 1, 64, 64, 0, 0.125, None) == -1
    assert lib.fa_base_softmax(GOOD, P(4098), GOOD, 1, 1, 64, 0, None) == -1
    assert lib.fa_base_softmax(GOOD, GOOD, GOOD, 1, 1, 16385, 0, None) == -2
    assert lib.fa_base_pv(GOOD, GOOD, None, 1, 1, 64, 64, 0, None) == -1
    assert lib.fa_base_softmax(GOOD, GOOD, GOOD, 1 << 16, 1 << 10, 1 << 6, 0, None) == -1   # B*H*N >= 2^31


def test_probe_argument_validation(lib):
    """The measured-ceiling probes check their arguments before any device work."""
    assert lib.fa_mfma_probe(None, 8, 3, None) == -1
    assert lib.fa_mfma_probe(GOOD, 0, 3, None) == -1
    assert lib.fa_mfma_probe(GOOD, 8, 0, None) == -1
    assert lib.fa_hbm_probe(GOOD, 100, P(1 << 20), None) == -1         # not a multiple of 16
    assert lib.fa_hbm_probe(GOOD, 256, None, None) == -1               # no sink
    assert lib.fa_hbm_probe(P(4100), 256, P(1 << 20), None) == -1      # misaligned
    assert lib.fa_issue_probe(-1, 1, GOOD, 4, 4, None) == -1           # kind outside 0..16
    assert lib.fa_issue_probe(17, 1, GOOD, 4, 4, None) == -1
    assert lib.fa_issue_probe(0, 3, GOOD, 4, 4, None) == -1            # one or two waves per SIMD
    assert lib.fa_issue_probe(7, 1, GOOD, 4, 4, None) == -1            # kind 7 pairs two waves
    assert lib.fa_issue_probe(0, 1, None, 4, 4, None) == -1
    assert lib.fa_issue_probe(0, 1, P(4098), 4, 4, None) == -1         # misaligned
    assert lib.fa_issue_probe(0, 1, GOOD, 0, 4, None) == -1
    assert lib.fa_issue_probe(0, 1, GOOD, 4, 0, None) == -1
    import torch
    if not torch.cuda.is_available():
        assert lib.fa_mfma_probe(GOOD, 8, 3, None) == -5
        assert lib.fa_hbm_probe(GOOD, 256, P(1 << 20), None) == -5
        assert lib.fa_issue_probe(7, 2, GOOD, 4, 4, None) == -5


def test_header_is_plain_c_and_links(lib, tmp_path):
    """include/fa.h is a C header: a C99 program that takes the address of
    every declared entry point compiles with gcc and links against libfa.so,
    and a forward call made from C with an invalid size returns
    FA_ERR_INVALID_ARG (checked before any device work, so the call never
    reaches a GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    names = _declared()
    src = tmp_path / "abi.c"
    src.write_text(
        "#include <stdio.h>\n#include \"fa.h\"\n"
        "int main(void) {\n"
        "  void* fns[] = {" + ", ".join(f"(void*){n}" for n in names) + "};\n"
        "  int st = fa_fwd((void*)4096, (void*)4096, (void*)4096, (void*)4096, (float*)4096,\n"
        "                  1, 1, 0, 64, 0, 0.125f, 0, 0);\n"
        "  printf(\"%d %d %s\\n\", (int)(sizeof(fns) / sizeof(fns[0])), st, fa_status_string(st));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "abi"
    libdir = os.path.dirname(fa.lib_path())
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", libdir, "-lfa", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    count, status = (int(x) for x in out.stdout.split()[:2])
    assert count == len(names)
    assert status == -1
