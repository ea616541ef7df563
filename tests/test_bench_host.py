"""Host-side parsing in bench.py: the power and clock readings it takes from amd-smi and
rocm-smi (text formats of ROCm 7.2's tools), checked on captured output without a GPU."""
import subprocess
import types

import bench

AMD_SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1381 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1900 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1880 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
"""

ROCM_SMI_TEXT = """======================================= Power Cap ========================================
GPU[0]		: Max Graphics Package Power (W): 1400.0
==========================================================================================
"""


def _fake_run(text):
    def run(cmd, **kw):
        return types.SimpleNamespace(stdout=text, stderr="", returncode=0)
    return run


def test_smi_sample_reads_power_and_mean_gfx_clock(monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_run(AMD_SMI_TEXT))
    pw, mhz = bench._smi_sample()
    assert pw == 1381.0
    assert mhz == 1890.0      # mean of the GFX clocks; the memory clock is not among them


def test_smi_sample_missing_fields(monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_run("GPU: 0\n    POWER:\n        N/A\n"))
    assert bench._smi_sample() is None

    def missing(cmd, **kw):
        raise FileNotFoundError(cmd[0])
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench._smi_sample() is None


def test_power_cap(monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_run(ROCM_SMI_TEXT))
    assert bench._power_cap() == 1400.0
