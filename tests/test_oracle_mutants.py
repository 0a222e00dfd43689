"""Mutation check of the oracle pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/hsw_oracle.c,
rebuilds that copy in a temporary directory and runs the pin suite against
it; the pins must fail.  This shows that the pins constrain the oracle's
formula rather than restate it.  The real oracle is never modified.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("sink dropped from the denominator",
     "double z = has_sink ? exp(sink - m) : 0.0;", "double z = 0.0;"),
    ("value scale ignored",
     "o[e] += p * (lambda * vrows[j][e]);", "o[e] += p * (vrows[j][e]);"),
    ("window one position too long",
     "int64_t lo = window > 0 ? p - window + 1 : 0;\n                if (lo < 0) lo = 0;\n                int64_t n",
     "int64_t lo = window > 0 ? p - window : 0;\n                if (lo < 0) lo = 0;\n                int64_t n"),
    ("rotation sign flipped",
     "yr[i] = xr[i] * c - xr[i + half] * s;", "yr[i] = xr[i] * c + xr[i + half] * s;"),
    ("GQA head mapping interleaved",
     "int g = h / group;\n                int64_t P", "int g = h % hkv;\n                int64_t P"),
    ("frequency base over the full head width",
     "inv_freq[i] = pow(theta, -2.0 * (double)i / (double)rope_dim);",
     "inv_freq[i] = pow(theta, -2.0 * (double)i / 192.0);"),
    ("ring slot position off by one",
     "int64_t held = P - back;", "int64_t held = P - back - 1;"),
    ("sink folded into a partial without its denominator term",
     "l[i] = l[i] * r + exp(sink[i] - mn);", "l[i] = l[i] * r;"),
    ("log-sum-exp merge without rescaling l",
     "z += w * l[c * n + i];", "z += l[c * n + i];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    for d in ("oracle", "tests", "hybrid_sliding_window_amd"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "_build", "csrc", "*.o"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path / "pytest.ini")
    src = tmp_path / "oracle" / "hsw_oracle.c"
    text = src.read_text()
    assert text.count(old) >= 1, f"mutation site not found: {old!r}"
    src.write_text(text.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
