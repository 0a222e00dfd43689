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
     "z[h] = sinks ? exp(sinks[h] - m[h]) : 0.0;", "z[h] = 0.0;"),
    ("value scale ignored",
     "oh[e] += p * (lambda * vrows[j][e]);", "oh[e] += p * (vrows[j][e]);"),
    ("sink also added to the numerator",
     "for (int h = 0; h < group; ++h) {\n        for (int e = 0; e < dv; ++e) o[h * (int64_t)dv + e] /= z[h];",
     "for (int h = 0; h < group; ++h) {\n        if (sinks) for (int e = 0; e < dv; ++e) "
     "o[h * (int64_t)dv + e] += exp(sinks[h] - m[h]);\n        for (int e = 0; e < dv; ++e) o[h * (int64_t)dv + e] /= z[h];"),
    ("each head's logits summed over the wrong query head",
     "for (int e = 0; e < dqk; ++e) qt[e * group + h] = q[h * (int64_t)dqk + e];",
     "for (int e = 0; e < dqk; ++e) qt[e * group + h] = q[((h + 1) % group) * (int64_t)dqk + e];"),
    ("window one position too long",
     "int64_t lo = window > 0 ? p - window + 1 : 0;", "int64_t lo = window > 0 ? p - window : 0;"),
    ("window one position too short",
     "int64_t lo = window > 0 ? p - window + 1 : 0;", "int64_t lo = window > 0 ? p - window + 2 : 0;"),
    ("rotation sign flipped",
     "yr[i] = xr[i] * c - xr[i + half] * s;", "yr[i] = xr[i] * c + xr[i + half] * s;"),
    ("GQA: a group of query heads reads the next KV head",
     "kr[j] = k + (row * hkv + g) * (int64_t)dqk;\n                    vr[j] = v + (row * hkv + g) * (int64_t)dv;",
     "kr[j] = k + (row * hkv + (g + 1) % hkv) * (int64_t)dqk;\n"
     "                    vr[j] = v + (row * hkv + (g + 1) % hkv) * (int64_t)dv;"),
    ("GQA in the ring decode: a group reads the next KV head's ring",
     "kr[n] = kring + ((s * hkv + g) * slots + t) * (int64_t)dqk;",
     "kr[n] = kring + ((s * hkv + (g + 1) % hkv) * slots + t) * (int64_t)dqk;"),
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
