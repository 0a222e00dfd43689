"""Independent brute-force formulation of the attention core, for tiny shapes.

Written separately from the oracle, with a different formulation of every
step, so that a mistake in one does not hide in the other:

- RoPE as complex multiplication: the pair (x[i], x[i+R/2]) is the complex
  number x[i] + 1j*x[i+R/2], multiplied by exp(1j * pos * theta**(-2i/R))
  (the rotate-half convention; colibri "What the engine implements").
- Attention as an explicit [T, T] boolean mask and a softmax over the
  concatenated row [sink, l_0, ..., l_{T-1}] with the sink's value row zero,
  so the sink joins the denominator and nothing else (colibri "What the
  engine implements"; gaudi-cookbook "What was built": the window is exactly
  the last 128 positions).
- GQA by explicitly repeating each KV head over its query heads.
"""
from __future__ import annotations

import numpy as np


def rope_complex(x: np.ndarray, pos: np.ndarray, theta: float, rope_dim: int) -> np.ndarray:
    x = np.asarray(x, np.float64)
    half = rope_dim // 2
    i = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * i / rope_dim)
    ang = np.asarray(pos, np.float64)[:, None] * freq[None, :]          # [T, half]
    z = x[..., :half] + 1j * x[..., half:rope_dim]                        # [T, H, half]
    z = z * np.exp(1j * ang)[:, None, :]
    y = x.copy()
    y[..., :half] = z.real
    y[..., half:rope_dim] = z.imag
    return y


def window_mask(qpos: np.ndarray, kpos: np.ndarray, window: int | None) -> np.ndarray:
    """allowed[i, j]: key at kpos[j] is visible to the query at qpos[i]."""
    qp = np.asarray(qpos)[:, None]
    kp = np.asarray(kpos)[None, :]
    allowed = kp <= qp
    if window is not None:
        allowed &= kp > qp - window
    return allowed


def attention(q, qpos, k, v, kpos, *, window, tau, lam, sinks=None):
    """q [nq, Hq, Dqk], k [nk, Hkv, Dqk], v [nk, Hkv, Dv]; window None = full."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, hq, _ = q.shape
    nk, hkv, _ = k.shape
    rep = hq // hkv
    kx = np.repeat(k, rep, axis=1)            # explicit MHA copy of each KV head
    vx = np.repeat(v, rep, axis=1) * lam
    allowed = window_mask(qpos, kpos, window)
    out = np.zeros((nq, hq, v.shape[2]))
    for h in range(hq):
        logits = tau * (q[:, h, :] @ kx[:, h, :].T)                       # [nq, nk]
        logits = np.where(allowed, logits, -np.inf)
        sink_col = np.full((nq, 1), -np.inf if sinks is None else float(sinks[h]))
        row = np.concatenate([sink_col, logits], axis=1)                  # [nq, 1+nk]
        mx = row.max(axis=1, keepdims=True)
        e = np.exp(row - mx)
        w = e / e.sum(axis=1, keepdims=True)
        vals = np.concatenate([np.zeros((1, vx.shape[2])), vx[:, h, :]], axis=0)
        out[:, h, :] = w @ vals
    return out


# ---------------------------------------------------------------- vision (ViT)
# The ViT step in another formulation (colibri "MiMo-V2.6 (Xiaomi)", the
# "vision" entry): 2D RoPE as complex multiplication with one frequency table
# per axis; the window blocks as a [T, T] boolean mask built from each
# token's position in the block's order.
def rope2d_complex(x: np.ndarray, row: np.ndarray, col: np.ndarray, theta: float) -> np.ndarray:
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half, quarter = d // 2, d // 4
    f = theta ** (-np.arange(quarter, dtype=np.float64) / quarter)
    ang = np.concatenate([np.asarray(row, np.float64)[:, None] * f[None, :],
                          np.asarray(col, np.float64)[:, None] * f[None, :]], axis=1)   # [T, half]
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def vit_mask(n: int, window: int, order=None, sink_key: bool = False) -> np.ndarray:
    """allowed[i, j] for picture-local tokens i (query) and j (key)."""
    order = np.arange(n) if order is None else np.asarray(order)
    where = np.empty(n, np.int64)
    where[order] = np.arange(n)           # token -> its position in the order
    if window == 0:
        return np.ones((n, n), bool)
    allowed = (where[:, None] // window) == (where[None, :] // window)
    if sink_key:
        allowed |= (where[None, :] == 0)
    return allowed


def vit_attention_masked(q, k, v, allowed, tau, sinks=None):
    """Softmax attention of one picture under a [T, T] mask, GQA by explicit
    repetition, the learned sink as an extra logit column with a zero value."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    T, hq, _ = q.shape
    hkv = k.shape[1]
    kk = np.repeat(k, hq // hkv, axis=1)
    vv = np.repeat(v, hq // hkv, axis=1)
    out = np.empty((T, hq, v.shape[2]))
    for h in range(hq):
        s = tau * q[:, h, :] @ kk[:, h, :].T
        s = np.where(allowed, s, -np.inf)
        if sinks is not None:
            s = np.concatenate([np.full((T, 1), sinks[h]), s], axis=1)
            vals = np.concatenate([np.zeros((1, v.shape[2])), vv[:, h, :]], axis=0)
        else:
            vals = vv[:, h, :]
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ vals
    return out
