"""Host logic of bench.py that needs no GPU: parsing amd-smi's power and clock
report, the refusal of more than one GPU, and the rule that the committed
counter figures count only for the kernel sources they were taken on."""
import subprocess
import sys
import types

import pytest

import bench

SMI = """GPU: 0
    POWER:
        SOCKET_POWER: 1377 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1900 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1910 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_smi_sample_parses_power_and_mean_gfx_clock(monkeypatch):
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: types.SimpleNamespace(stdout=SMI, returncode=0))
    assert bench._smi_sample() == (1377.0, 1905.0)   # the memory clock is not averaged in


def test_smi_sample_without_the_tool(monkeypatch):
    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench._smi_sample() == (None, None)
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: types.SimpleNamespace(stdout="", returncode=1))
    assert bench._smi_sample() == (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_counter_figures_follow_the_kernel_sources(tmp_path, monkeypatch):
    """The committed counter summaries are reported only while the kernel
    sources they were taken on are unchanged; comments and spacing do not
    count as a change."""
    csrc = tmp_path / "precision_numerics_fa_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for name in bench.KERNEL_SOURCES:
        (csrc / name).write_text("int f(int x) { return x + 1; }  // add one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest()
    rec = {"source_digest": digest, "kernels": {"fwd_kernel": {"hbm_bytes_per_launch": 123}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(bench.json.dumps(rec))
    assert bench.counter_traffic("fwd_kernel") == 123
    assert bench.counter_traffic("bwd_grads_kernel") is None
    # a comment-only edit keeps the figures
    (csrc / bench.KERNEL_SOURCES[0]).write_text("/* note */ int f(int x) {\n  return x + 1;\n}\n")
    assert bench.source_digest() == digest and bench.counter_traffic("fwd_kernel") == 123
    # a code edit retires them
    (csrc / bench.KERNEL_SOURCES[0]).write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest() != digest and bench.counter_traffic("fwd_kernel") is None
