"""Pins of the oracle's vision-encoder (ViT) functions, against what the page
and the mathematics fix (colibri "MiMo-V2.6 (Xiaomi)", the model
description's "vision" entry: 2D RoPE, grouped-query attention, full
attention in some blocks and a 1D window of 64 tokens in the others, row and
column order of the 2x2 merge units alternating, a sink on the first key of
the window blocks).

- layout: hand-worked grids and the invariants of the two unit orders;
- 2D RoPE: closed forms (the slowest frequency turns by exactly the row or
  the column), axis separation, norms, and the complex-number formulation of
  tests/brute.py;
- attention: a textbook softmax (numpy matmul) for whole pictures and for
  each window, the [T, T] mask formulation of tests/brute.py for the orders
  and the sink key, and the degenerate cases (one window covering the
  picture is full attention; pictures do not see each other).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from brute import rope2d_complex, vit_attention_masked, vit_mask


def rng(seed):
    return np.random.default_rng(seed)


def textbook(q, k, v, tau):
    """softmax(tau q k^T) v per head, GQA by repetition (numpy matmul)."""
    hq, hkv = q.shape[1], k.shape[1]
    out = np.empty((q.shape[0], hq, v.shape[2]))
    for h in range(hq):
        s = tau * q[:, h] @ k[:, h // (hq // hkv)].T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = (p / p.sum(axis=1, keepdims=True)) @ v[:, h // (hq // hkv)]
    return out


# ------------------------------------------------------------------ layout
def test_layout_by_hand_4x4():
    row, col, co = oracle.vit_layout(4, 4)
    # units (0,0), (0,1), (1,0), (1,1); each TL, TR, BL, BR
    assert row.tolist() == [0, 0, 1, 1, 0, 0, 1, 1, 2, 2, 3, 3, 2, 2, 3, 3]
    assert col.tolist() == [0, 1, 0, 1, 2, 3, 2, 3, 0, 1, 0, 1, 2, 3, 2, 3]
    # column order walks units (0,0), (1,0), (0,1), (1,1)
    assert co.tolist() == [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]


def test_layout_by_hand_2x6():
    row, col, co = oracle.vit_layout(2, 6)
    assert row.tolist() == [0, 0, 1, 1] * 3
    assert col.tolist() == [0, 1, 0, 1, 2, 3, 2, 3, 4, 5, 4, 5]
    assert co.tolist() == list(range(12))        # one unit row: both orders agree


@pytest.mark.parametrize("h,w", [(8, 6), (28, 36), (2, 2), (64, 64)])
def test_layout_invariants(h, w):
    row, col, co = oracle.vit_layout(h, w)
    n = h * w
    assert sorted(zip(row.tolist(), col.tolist())) == [(r, c) for r in range(h) for c in range(w)]
    assert sorted(co.tolist()) == list(range(n))
    for t in range(0, n, 4):                     # each unit is a 2x2 square, TL TR BL BR
        assert (row[t:t + 4] - row[t]).tolist() == [0, 0, 1, 1] and (col[t:t + 4] - col[t]).tolist() == [0, 1, 0, 1]
        assert row[t] % 2 == 0 and col[t] % 2 == 0
    ur, uc = row[::4] // 2, col[::4] // 2        # row order: unit row major
    assert np.all(np.diff(ur * (w // 2) + uc) == 1)
    cur, cuc = row[co][::4] // 2, col[co][::4] // 2  # column order: unit column major
    assert np.all(np.diff(cuc * (h // 2) + cur) == 1)
    assert co[0] == 0                            # both orders start at the same token
    with pytest.raises(ValueError):
        oracle.vit_layout(3, 4)


# ----------------------------------------------------------------- 2D RoPE
def test_rope2d_slowest_frequency_turns_by_row_and_col():
    d = 64
    x = np.zeros((3, 1, d))
    x[:, 0, 0] = 1.0             # pair (0, 32): frequency 1, row axis
    row = np.array([0, 5, 37], np.int32)
    col = np.array([9, 2, 11], np.int32)
    y = oracle.rope_2d(x, row, col, 1e4)
    assert np.allclose(y[:, 0, 0], np.cos(row)) and np.allclose(y[:, 0, 32], np.sin(row))
    assert np.count_nonzero(np.abs(y) > 1e-15) <= 6
    x2 = np.zeros((3, 1, d))
    x2[:, 0, 16] = 1.0           # pair (16, 48): frequency 1, column axis
    y2 = oracle.rope_2d(x2, row, col, 1e4)
    assert np.allclose(y2[:, 0, 16], np.cos(col)) and np.allclose(y2[:, 0, 48], np.sin(col))
    x3 = np.zeros((1, 1, d))
    x3[0, 0, 8] = 1.0            # pair (8, 40): theta^(-8/16) = 1e-2 for theta 1e4
    y3 = oracle.rope_2d(x3, np.array([100], np.int32), np.array([0], np.int32), 1e4)
    assert np.isclose(y3[0, 0, 8], np.cos(1.0)) and np.isclose(y3[0, 0, 40], np.sin(1.0))


def test_rope2d_axes_separate_and_norms_kept():
    g = rng(1)
    x = g.standard_normal((50, 4, 64))
    row = g.integers(0, 100, 50).astype(np.int32)
    col = g.integers(0, 100, 50).astype(np.int32)
    y = oracle.rope_2d(x, row, col, 1e4)
    # changing the column leaves the row pairs (i < 16 and i + 32) untouched
    y2 = oracle.rope_2d(x, row, col + 7, 1e4)
    idx = np.r_[0:16, 32:48]
    assert np.array_equal(y[..., idx], y2[..., idx]) and not np.allclose(y, y2)
    pair = lambda z: z[..., :32] ** 2 + z[..., 32:] ** 2
    assert np.allclose(pair(y), pair(x))
    zero = oracle.rope_2d(x, np.zeros(50, np.int32), np.zeros(50, np.int32), 1e4)
    assert np.array_equal(zero, x)


def test_rope2d_matches_complex_formulation_and_is_relative():
    g = rng(2)
    q = g.standard_normal((40, 2, 64))
    k = g.standard_normal((40, 2, 64))
    row = g.integers(0, 64, 40).astype(np.int32)
    col = g.integers(0, 64, 40).astype(np.int32)
    assert np.allclose(oracle.rope_2d(q, row, col, 1e4), rope2d_complex(q, row, col, 1e4), atol=1e-12)
    # <R(a) q, R(b) k> depends on a - b only (both axes)
    a = oracle.rope_2d(q, row, col, 1e4)
    b = oracle.rope_2d(k, row[::-1].copy(), col[::-1].copy(), 1e4)
    a2 = oracle.rope_2d(q, row + 13, col + 4, 1e4)
    b2 = oracle.rope_2d(k, row[::-1] + 13, col[::-1] + 4, 1e4)
    assert np.allclose(np.einsum("thd,thd->th", a, b), np.einsum("thd,thd->th", a2, b2))


# --------------------------------------------------------------- attention
TAU = 1 / 8.0


def picture(g, n, hq=4, hkv=2, d=64):
    return (g.standard_normal((n, hq, d)), g.standard_normal((n, hkv, d)), g.standard_normal((n, hkv, d)))


@pytest.mark.parametrize("n,hq,hkv", [(1, 4, 2), (37, 4, 1), (130, 8, 2)])
def test_full_picture_is_textbook_attention(n, hq, hkv):
    q, k, v = picture(rng(3), n, hq, hkv)
    got = oracle.vit_attn(q, k, v, [0, n], window=0, tau=TAU)
    assert np.allclose(got, textbook(q, k, v, TAU), atol=1e-12)


@pytest.mark.parametrize("n", [64, 100, 192, 200])
def test_windows_in_row_order_are_textbook_per_window(n):
    q, k, v = picture(rng(4), n)
    got = oracle.vit_attn(q, k, v, [0, n], window=64, tau=TAU)
    for lo in range(0, n, 64):
        hi = min(n, lo + 64)
        assert np.allclose(got[lo:hi], textbook(q[lo:hi], k[lo:hi], v[lo:hi], TAU), atol=1e-12)


def test_sink_key_is_the_first_token_in_each_window():
    n = 150
    q, k, v = picture(rng(5), n)
    got = oracle.vit_attn(q, k, v, [0, n], window=64, tau=TAU, sink_key=True)
    assert np.allclose(got[:64], textbook(q[:64], k[:64], v[:64], TAU), atol=1e-12)   # held once
    for lo in (64, 128):
        hi = min(n, lo + 64)
        kk = np.concatenate([k[:1], k[lo:hi]])
        vv = np.concatenate([v[:1], v[lo:hi]])
        assert np.allclose(got[lo:hi], textbook(q[lo:hi], kk, vv, TAU), atol=1e-12)


@pytest.mark.parametrize("h,w,sink_key,learned", [(8, 12, True, False), (16, 10, False, True),
                                                  (14, 18, True, True), (2, 40, True, False)])
def test_column_order_against_mask_formulation(h, w, sink_key, learned):
    g = rng(6)
    n = h * w
    q, k, v = picture(g, n, 4, 2)
    sinks = g.standard_normal(4) if learned else None
    _, _, co = oracle.vit_layout(h, w)
    for order in (None, co):
        got = oracle.vit_attn(q, k, v, [0, n], window=64, tau=TAU, order=order, sink_key=sink_key,
                              sinks=sinks)
        ref = vit_attention_masked(q, k, v, vit_mask(n, 64, order, sink_key), TAU, sinks)
        assert np.allclose(got, ref, atol=1e-12)


def test_one_window_over_the_picture_is_full_attention():
    q, k, v = picture(rng(7), 60)
    full = oracle.vit_attn(q, k, v, [0, 60], window=0, tau=TAU)
    win = oracle.vit_attn(q, k, v, [0, 60], window=64, tau=TAU, sink_key=True)
    assert np.allclose(win, full, atol=1e-13)


def test_pictures_do_not_see_each_other_and_order_is_per_picture():
    g = rng(8)
    q, k, v = picture(g, 96 + 40)
    cu = [0, 96, 136]
    _, _, co = oracle.vit_layout(8, 12)
    order = np.concatenate([co, np.arange(40)]).astype(np.int32)
    a = oracle.vit_attn(q, k, v, cu, window=64, tau=TAU, order=order, sink_key=True)
    k2, v2 = k.copy(), v.copy()
    k2[96:] += 3.0
    v2[96:] -= 1.0
    b = oracle.vit_attn(q, k2, v2, cu, window=64, tau=TAU, order=order, sink_key=True)
    assert np.array_equal(a[:96], b[:96]) and not np.allclose(a[96:], b[96:])
    alone = oracle.vit_attn(q[:96], k[:96], v[:96], [0, 96], window=64, tau=TAU, order=co, sink_key=True)
    assert np.array_equal(a[:96], alone)
    with pytest.raises(ValueError):
        oracle.vit_attn(q, k, v, cu, window=64, tau=TAU, order=np.full(136, 96, np.int32))


def test_any_order_and_its_first_token_as_sink_against_mask_formulation():
    """An arbitrary permutation (not starting at token 0): the windows follow
    it and the sink key is the token it puts first."""
    g = rng(9)
    n = 170
    q, k, v = picture(g, n, 8, 2)
    order = g.permutation(n).astype(np.int32)
    assert order[0] != 0
    got = oracle.vit_attn(q, k, v, [0, n], window=64, tau=TAU, order=order, sink_key=True)
    ref = vit_attention_masked(q, k, v, vit_mask(n, 64, order, True), TAU)
    assert np.allclose(got, ref, atol=1e-12)
