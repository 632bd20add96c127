"""Host-side pieces of bench.py: the launch-duration statistics, the amd-smi
reading behind ``--power``, and the refusal of more than one GPU.  No GPU
is used."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# amd-smi metric -p -c output, shortened to two of the eight graphics
# partitions (one per XCD) and with one partition's clock not reported
SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1391 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1824 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1776 MHz
            MIN_CLK: 500 MHz
        GFX_2:
            CLK: N/A
        MEM_0:
            CLK: 2000 MHz
"""


def _fake_run(text, rc=0):
    def run(cmd, **kw):
        assert cmd[:2] == ["amd-smi", "metric"]
        return types.SimpleNamespace(stdout=text, stderr="", returncode=rc)
    return run


def test_smi_sample_reads_power_and_mean_graphics_clock(monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_run(SMI_TEXT))
    r = bench.smi_sample(0)
    assert r["socket_power_w"] == 1391.0
    # the memory clock and the unreported partition are left out
    assert r["gfx_clocks_mhz"] == [1824.0, 1776.0]
    assert r["gfx_clock_mhz"] == 1800.0


def test_smi_sample_reports_a_missing_tool(monkeypatch):
    def run(cmd, **kw):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", run)
    assert "error" in bench.smi_sample(0)
    monkeypatch.setattr(subprocess, "run", _fake_run("no devices\n", rc=1))
    assert "error" in bench.smi_sample(0)


def test_launch_stats_percentiles():
    ms = np.arange(1, 101) / 1000.0  # 1 .. 100 us
    s = bench.launch_stats(ms)
    assert s["kernel_mean_us"] == pytest.approx(50.5)
    assert s["kernel_median_us"] == pytest.approx(50.5)
    assert s["kernel_p10_us"] == pytest.approx(10.9)
    assert s["kernel_p90_us"] == pytest.approx(90.1)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
