"""Host logic of bench.py that needs no GPU: parsing amd-smi's power and clock
report, and the refusal of more than one GPU."""
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
