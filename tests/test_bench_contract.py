"""bench.py's contract on the host (no GPU): one GPU only, the own-roofline
arithmetic of every call, and the counter-measured traffic reported only for
the kernel sources it was measured on."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_own_roofline_fraction():
    d = bench.own_roofline(dict(ms=2.0, flops=5.0e12, bytes=8.0e9, tokens=1000))
    assert d["roofline_bound"] == "mfma"                  # 2 ms of MFMA work against 1 ms of HBM
    assert d["roofline_frac"] == pytest.approx(1.0)
    assert d["tokens_per_s"] == pytest.approx(5.0e5)
    d = bench.own_roofline(dict(ms=4.0, bytes=16.0e9))
    assert d["roofline_bound"] == "hbm" and d["roofline_frac"] == pytest.approx(0.5)
    assert "roofline_frac" not in bench.own_roofline(dict(ms=1.0))
    nan = bench.own_roofline(dict(ms=float("nan"), bytes=1.0))
    assert "roofline_frac" not in nan


def test_measured_traffic_is_the_stored_bytes_or_null():
    for call, (nbytes, files, digest) in bench.MEASURED_TRAFFIC.items():
        got = bench.measured_traffic(call)
        assert got in (nbytes, None), call
        for f in files:
            assert os.path.exists(os.path.join(bench.CSRC, f)), f
