"""Comparison metrics shared by the parity tests.

max_abs  = max_k |y_k - r_k|
mean_rel = sum_k |y_k - r_k| / sum_k |r_k|   (L1 ratio over all outputs of a call;
           an elementwise mean of |dy|/|r| is meaningless where outputs sit
           near zero, as they do when the sink takes almost all the mass)
"""
from __future__ import annotations

import numpy as np

MAX_ABS_BAR = 2e-2
MEAN_REL_BAR = 2e-3


def errors(y, r):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    d = np.abs(y - r)
    denom = np.abs(r).sum()
    return float(d.max()) if d.size else 0.0, float(d.sum() / denom) if denom > 0 else float(d.sum())


def assert_close(y, r, max_abs=MAX_ABS_BAR, mean_rel=MEAN_REL_BAR, what=""):
    ma, mr = errors(y, r)
    assert np.all(np.isfinite(np.asarray(y, np.float64))), f"{what}: non-finite output"
    assert ma <= max_abs and mr <= mean_rel, f"{what}: max_abs={ma:.3e} (bar {max_abs}) mean_rel={mr:.3e} (bar {mean_rel})"
    return ma, mr
