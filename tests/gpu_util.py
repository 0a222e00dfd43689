"""Helpers for the GPU parity tests: calls through the C ABI on cuda:0 and
builds the oracle's inputs from the exact tensors each call consumed."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from hybrid_sliding_window_amd import workloads as wl

DEV = "cuda:0"


def note(msg: str):
    """Name the case on stdout before a GPU step, flushed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """One unit in the last place of bf16 at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def linear_kv_from_ring(kring_s, vring_s, start: int, kstage, vstage, window=128):
    """K/V laid out by position from max(0, start-window+1) through the chunk:
    prior positions read from ring slot p mod window, the chunk from staging.
    kring_s [Hkv, W, D] fp64, kstage [T, Hkv, D] fp64.  Returns (k, v, kpos0)."""
    lo = max(0, start - window + 1)
    ks = [kring_s[:, p % window, :] for p in range(lo, start)]
    vs = [vring_s[:, p % window, :] for p in range(lo, start)]
    k = np.concatenate([np.stack(ks), kstage], axis=0) if ks else kstage
    v = np.concatenate([np.stack(vs), vstage], axis=0) if vs else vstage
    return k, v, lo


def shape_kw(shape):
    return dict(tau=shape.softmax_scale, lam=shape.value_scale)
