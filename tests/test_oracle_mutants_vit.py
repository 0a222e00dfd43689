"""Mutation check of the vision-attention oracle pins (CPU only).

Each case plants one plausible mistake in the vision part of a copy of
oracle/hsw_oracle.c (token layout, 2D RoPE, windowed attention with the sink
key), rebuilds that copy in a temporary directory and runs
tests/test_oracle_pins_vit.py against it; the pins must fail.  This shows
that the vision pins constrain the oracle's formulas (colibri "MiMo-V2.6
(Xiaomi)", the vision entry: 2D RoPE, 1D windows of 64 tokens in alternating
row and column order of the 2x2 merge units, a sink on the first key of the
window blocks) rather than restate them.  The real oracle is never modified.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("2D RoPE row and column axes swapped",
     "double coord = i < quarter ? (double)row[t] : (double)col[t];",
     "double coord = i < quarter ? (double)col[t] : (double)row[t];"),
    ("2D RoPE frequency exponent doubled",
     "double a = coord * pow(theta, -(double)f / (double)quarter);",
     "double a = coord * pow(theta, -2.0 * (double)f / (double)quarter);"),
    ("2D RoPE rotation sign flipped",
     "yr[i] = xr[i] * c - xr[i + half] * s;\n                yr[i + half] = xr[i + half] * c + xr[i] * s;\n"
     "            }\n            for (int e = 2 * half",
     "yr[i] = xr[i] * c + xr[i + half] * s;\n                yr[i + half] = xr[i + half] * c - xr[i] * s;\n"
     "            }\n            for (int e = 2 * half"),
    ("merge unit patches taken column-major (TL, BL, TR, BR)",
     "row[t] = 2 * (u / uw) + e / 2;\n        col[t] = 2 * (u % uw) + e % 2;",
     "row[t] = 2 * (u / uw) + e % 2;\n        col[t] = 2 * (u % uw) + e / 2;"),
    ("column order equal to row order",
     "col_order[j] = 4 * (ur * uw + ucl) + j % 4;",
     "col_order[j] = 4 * uc + j % 4;"),
    ("column order walks units with the grid's sides swapped",
     "int ur = uc % uh, ucl = uc / uh;",
     "int ur = uc % uw, ucl = uc / uw;"),
    ("sink key dropped",
     "if (sink_key && lo > 0) {",
     "if (0 && sink_key && lo > 0) {"),
    ("sink key taken from the picture's second token",
     "int64_t r0 = base + (order ? order[base] : 0);",
     "int64_t r0 = base + (order ? order[base + 1] : 1);"),
    ("sink key taken in row order instead of the block's order",
     "int64_t r0 = base + (order ? order[base] : 0);",
     "int64_t r0 = base;"),
    ("a window's last key dropped",
     "hi = lo + window < n ? lo + window : n;",
     "hi = lo + window < n ? lo + window - 1 : n - 1;"),
    ("windows cut in row order whatever the block's order",
     "int64_t r = base + (order ? order[base + jj] : jj);",
     "int64_t r = base + jj;"),
    ("GQA head mapping interleaved in the vision attention",
     "int h = (int)(jh % hq), g = h / group;",
     "int h = (int)(jh % hq), g = h % hkv;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_vit_pins_catch_planted_mistake(tmp_path, name, old, new):
    for d in ("oracle", "tests", "hybrid_sliding_window_amd"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "_build", "csrc", "*.o"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path / "pytest.ini")
    src = tmp_path / "oracle" / "hsw_oracle.c"
    text = src.read_text()
    assert text.count(old) == 1, f"mutation site not found once: {old!r}"
    src.write_text(text.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins_vit.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"vision pins did not catch: {name}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
