"""Pins for the fp64 oracle: checks against what the pages and mathematics fix,
never against the oracle's own formula retyped.

Each test names the property it pins and the passage it comes from.  Together
they are chosen so that a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle fails at least one of them:

  sink in numerator / dropped / scaled ........ P1, P6, P12, P13
  window off by one, wrong ring position ...... P4, P6, P12, golden slot rule
  rotation sign / pairing / frequency base ..... P6 (complex formulation), P8
  GQA head mapping ............................. P6 (explicit repeat), P9
  value scale .................................. P6, P11, P12, P13
  softmax merge / split-K ...................... P5, P7
  full attention ............................... P2 (library routine)
"""
from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
import brute
from hybrid_sliding_window_amd import workloads as wl
from parity import errors

TAU = 1.0 / math.sqrt(192.0)
LAM = 0.707
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def rng(seed):
    return np.random.default_rng(seed)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


# ---------------------------------------------------------------- P1 sink
def test_p1_sink_joins_denominator_only():
    """colibri 'What the engine implements': the sink joins the softmax
    denominator and nothing else.  With S = exp(lse_nosink):
    o_sink = o_nosink * S / (S + e^sigma)."""
    d = wl.logit_shift_layer(n_tok=256)
    q, k, v = (d[n].double().numpy() for n in "qkv")
    pos = d["pos"].numpy()
    s = d["sinks"].double().numpy()
    kw = dict(window=128, tau=TAU, lam=LAM)
    o0, lse0 = oracle.attn_linear(q, pos, k, v, 0, want_lse=True, **kw)
    o1 = oracle.attn_linear(q, pos, k, v, 0, sinks=s, **kw)
    factor = 1.0 / (1.0 + np.exp(s[None, :] - lse0))        # S/(S+e^s)
    expect = o0 * factor[..., None]
    assert rel(o1, expect) < 1e-12


def test_p1_page_regime_sink_takes_almost_all_mass():
    """gaudi-cookbook 'What was built': logits near -25, sinks near +1, so the
    sink normally takes almost all the mass.  The workload reproduces those
    statistics; the oracle's sink mass must exceed 1 - 1e-5 in every row, and
    an attention that drops the sink (as the page says FusedSDPA does) is
    off by orders of magnitude, far outside the parity bar."""
    page = json.load(open(GOLDEN))["sink_regime"]
    d = wl.logit_shift_layer(n_tok=512)
    q, k, v = (d[n].double().numpy() for n in "qkv")
    pos = d["pos"].numpy()
    s = d["sinks"].double().numpy()
    # the workload's scaled logits inside the window (independent numpy)
    lg = TAU * np.einsum("thd,jd->thj", q, k[:, 0, :])
    mask = brute.window_mask(pos, pos, 128)
    vals = lg[np.broadcast_to(mask[:, None, :], lg.shape)]
    assert abs(vals.mean() - page["logit_mean"]) < 1.5 and 2.0 < vals.std() < 4.0
    assert abs(s.mean() - page["sink_mean"]) < 0.3
    kw = dict(window=128, tau=TAU, lam=LAM)
    _, lse0 = oracle.attn_linear(q, pos, k, v, 0, want_lse=True, **kw)
    mass = np.exp(s[None, :]) / (np.exp(s[None, :]) + np.exp(lse0))
    assert mass.min() > 1 - 1e-5
    o_sink = oracle.attn_linear(q, pos, k, v, 0, sinks=s, **kw)
    o_drop = oracle.attn_linear(q, pos, k, v, 0, **kw)
    _, mr = errors(o_drop, o_sink)
    assert mr > 1e3


# ------------------------------------------------- P2 window >= T = causal
@pytest.mark.parametrize("T,hq,hkv", [(37, 4, 1), (200, 8, 2)])
def test_p2_wide_window_no_sink_is_causal_attention(T, hq, hkv):
    """A window at least as long as the sequence with no sink is plain causal
    attention (full layers carry no sink: colibri 'What the engine
    implements').  Checked against torch's scaled_dot_product_attention in
    float64 on the CPU, and bitwise against the full-attention mode."""
    r = rng(11)
    q, k, v = r.standard_normal((T, hq, 192)), r.standard_normal((T, hkv, 192)), r.standard_normal((T, hkv, 128))
    pos = np.arange(T)
    ow = oracle.attn_linear(q, pos, k, v, 0, window=T + 5, tau=TAU, lam=LAM)
    of = oracle.attn_linear(q, pos, k, v, 0, window=0, tau=TAU, lam=LAM)
    assert np.array_equal(ow, of)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v * LAM).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=TAU)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert rel(of, ref) < 1e-12


# ------------------------------------------------------- P3 V zero-padding
def test_p3_zero_padded_v_changes_nothing():
    """gaudi-cookbook 'What was built': padding V from 128 to 192 with zeros is
    exact, since a zero V column adds nothing."""
    r = rng(3)
    T = 150
    q, k, v = r.standard_normal((T, 8, 192)), r.standard_normal((T, 2, 192)), r.standard_normal((T, 2, 128))
    s = 1 + 0.25 * r.standard_normal(8)
    vp = np.concatenate([v, np.zeros((T, 2, 64))], axis=2)
    pos = np.arange(T)
    o = oracle.attn_linear(q, pos, k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    op = oracle.attn_linear(q, pos, k, vp, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    assert np.array_equal(op[..., :128], o)
    assert np.all(op[..., 128:] == 0.0)


# ----------------------------------------------------------- P4 ring rule
@pytest.mark.parametrize("P", [0, 1, 50, 126, 127, 128, 129, 300, 1000])
def test_p4_ring_equals_linear_window(P):
    """colibri 'System One mode and prompt reuse': position p in slot p mod 128;
    gaudi-cookbook 'What was built': the window is exactly the last 128
    positions.  A ring filled slot = p mod 128 for p = 0..P and decoded at P
    equals attention over the linear window."""
    r = rng(40 + P)
    n = P + 1
    k, v = r.standard_normal((n, 2, 192)), r.standard_normal((n, 2, 128))
    q = r.standard_normal((1, 8, 192))
    s = 1 + 0.25 * r.standard_normal(8)
    kring = np.zeros((1, 2, 128, 192))
    vring = np.zeros((1, 2, 128, 128))
    for p in range(n):                    # later positions overwrite earlier
        kring[0, :, p % 128] = k[p]
        vring[0, :, p % 128] = v[p]
    od = oracle.ring_decode(q, [P], kring, vring, tau=TAU, lam=LAM, sinks=s)
    ol = oracle.attn_linear(q, [P], k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    assert rel(od, ol) < 1e-13


def test_p4_slot_and_row_indices_exact():
    """Integer destination rule: ring slot = p mod 128, pool row = base + p,
    staging row = t (colibri 'System One mode and prompt reuse')."""
    r = rng(5)
    ps = np.concatenate([np.arange(0, 300), r.integers(0, 2 ** 20 + 1, 2000), [2 ** 20]])
    for p in ps:
        assert oracle.dst_index(oracle.RING, 0, int(p)) == int(p) & 127
    assert oracle.dst_index(oracle.POOL, 3, 1000, seq_base=77777) == 78777
    assert oracle.dst_index(oracle.STAGING, 42, 123456) == 42


# ---------------------------------------------- P5 per-block sink - log n
@pytest.mark.parametrize("n", [1, 2, 3, 7, 64])
def test_p5_per_block_sink_minus_log_n_is_one_sink(n):
    """gaudi-cookbook 'What was built': each of a sequence's n blocks gets the
    sink minus log(n), so the n copies sum to one sink term."""
    r = rng(50 + n)
    L = 300
    q, k, v = r.standard_normal((1, 4, 192)), r.standard_normal((L, 1, 192)), r.standard_normal((L, 1, 128))
    s = 1 + 0.25 * r.standard_normal(4)
    cuts = np.sort(r.choice(np.arange(1, L), size=n - 1, replace=False)) if n > 1 else []
    edges = [0, *cuts, L]
    parts = [oracle.attn_partial(q, [L - 1], k, v, 0, a, b, window=0, tau=TAU, lam=LAM)
             for a, b in zip(edges[:-1], edges[1:])]
    joined = [oracle.join_sink(m, l, acc, (s - math.log(n))[None, :]) for m, l, acc in parts]
    o, lse = oracle.lse_merge(np.stack([j[0] for j in joined]), np.stack([j[1] for j in joined]),
                              np.stack([j[2] for j in joined]))
    ref, lse_ref = oracle.attn_linear(q, [L - 1], k, v, 0, window=0, tau=TAU, lam=LAM, sinks=s,
                                      want_lse=True)
    assert rel(o, ref) < 1e-13 and rel(lse, lse_ref) < 1e-13


# --------------------------------------------------- P6 brute force, tiny
CASES = [(T, W, hh, dd) for T in (1, 2, 3, 5, 127, 128, 129, 200)
         for W in (1, 2, 4, 128, None)
         for hh in ((1, 1), (4, 1), (8, 2))
         for dd in ((192, 128), (8, 4))]


@pytest.mark.parametrize("T,W,hh,dd", CASES)
def test_p6_brute_force_tiny(T, W, hh, dd):
    """Rope + attention of the oracle against the independent brute force
    (complex rotation, explicit mask, softmax over [sink, logits])."""
    hq, hkv = hh
    dqk, dv = dd
    R = min(64, dqk // 2 * 2)
    if dqk == 8:
        R = 4
    r = rng(T * 1000 + (W or 0) * 10 + hq + dqk)
    q, k, v = r.standard_normal((T, hq, dqk)), r.standard_normal((T, hkv, dqk)), r.standard_normal((T, hkv, dv))
    s = 1 + 0.25 * r.standard_normal(hq)
    theta = 1e4 if W is not None else 1e7
    # rotation at arbitrary absolute positions
    start = int(r.integers(0, 600000))
    pos = np.arange(start, start + T)
    qr, kr = oracle.rope(q, pos, theta, R), oracle.rope(k, pos, theta, R)
    bq, bk = brute.rope_complex(q, pos, theta, R), brute.rope_complex(k, pos, theta, R)
    # both sides round the angle pos * freq once in fp64 (freq may differ by
    # an ulp between libm pow and numpy), so the bound scales with the position
    tol = 1e-13 + 8.0 * (start + T) * 2.0 ** -53
    assert rel(qr, bq) < tol and rel(kr, bk) < tol
    tau = 1.0 / math.sqrt(dqk)
    sk = s if W is not None else None
    # attention over a sequence that starts at position 0 (so every key the
    # window or the causal prefix needs is present)
    pos0 = np.arange(T)
    qr0, kr0 = oracle.rope(q, pos0, theta, R), oracle.rope(k, pos0, theta, R)
    o = oracle.attn_linear(qr0, pos0, kr0, v, 0, window=W or 0, tau=tau, lam=LAM, sinks=sk)
    b = brute.attention(brute.rope_complex(q, pos0, theta, R), pos0,
                        brute.rope_complex(k, pos0, theta, R), v, pos0,
                        window=W, tau=tau, lam=LAM, sinks=sk)
    assert rel(o, b) < 1e-13


# ------------------------------------------------ P7 split-K LSE merge
def test_p7_splitk_merge_equals_unsplit():
    """Split-K decode partials merged by log-sum-exp equal the unsplit result
    for random partitions (gaudi-cookbook 'What was built': per-block decode)."""
    r = rng(7)
    L = 5000
    q, k, v = r.standard_normal((3, 16, 192)), r.standard_normal((L, 1, 192)), r.standard_normal((L, 1, 128))
    qpos = np.array([L - 1, 4000, 2047])
    for trial in range(5):
        n = int(r.integers(1, 12))
        edges = [0, *np.sort(r.choice(np.arange(1, L), size=n - 1, replace=False)), L]
        parts = [oracle.attn_partial(q, qpos, k, v, 0, a, b, window=0, tau=TAU, lam=LAM)
                 for a, b in zip(edges[:-1], edges[1:])]
        o, lse = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                                  np.stack([p[2] for p in parts]))
        ref, lse_ref = oracle.attn_linear(q, qpos, k, v, 0, window=0, tau=TAU, lam=LAM, want_lse=True)
        assert rel(o, ref) < 1e-13 and rel(lse, lse_ref) < 1e-13


# ------------------------------------------------------------ P8 RoPE
def test_p8_rope_identity_norms_passthrough_relative():
    r = rng(8)
    x = r.standard_normal((6, 3, 192))
    assert np.array_equal(oracle.rope(x, np.zeros(6, np.int64), 1e4), x)
    pos = np.array([1, 127, 128, 196608, 205000, 524288])
    y = oracle.rope(x, pos, 1e4)
    assert np.array_equal(y[..., 64:], x[..., 64:])
    n0 = x[..., :32] ** 2 + x[..., 32:64] ** 2
    n1 = y[..., :32] ** 2 + y[..., 32:64] ** 2
    assert np.abs(n1 - n0).max() <= 1e-14 * n0.max()
    # <R(q,p), R(k,p')> = <R(q,p-p'), k> at large positions, both thetas
    for theta in (1e4, 1e7):
        q = r.standard_normal((1, 1, 192))
        k = r.standard_normal((1, 1, 192))
        p, pp = 524287, 500000
        lhs = np.sum(oracle.rope(q, [p], theta) * oracle.rope(k, [pp], theta))
        rhs = np.sum(oracle.rope(q, [p - pp], theta) * k)
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


def test_p8_rope_angles_against_mpmath():
    """gaudi-cookbook 'The RoPE fix for large positions': angles must be right
    at large positions (device fp32 failed past ~1.5e5 rad).  Rotating unit
    vectors exposes cos/sin of every one of the 32 angles, compared with
    50-digit mpmath values of pos * theta^(-2i/64)."""
    mpmath.mp.dps = 50
    poss = [1, 127, 128, 196608, 200000, 205000, 262143, 524287, 524288]
    for theta in (1e4, 1e7):
        e = np.zeros((len(poss), 32, 192))
        for i in range(32):
            e[:, i, i] = 1.0
        y = oracle.rope(e, np.array(poss), theta)
        for a, p in enumerate(poss):
            for i in range(32):
                ang = mpmath.mpf(p) * mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / 64)
                assert abs(y[a, i, i] - float(mpmath.cos(ang))) < 1e-9
                assert abs(y[a, i, i + 32] - float(mpmath.sin(ang))) < 1e-9


def test_p8_page_values_cos_200000_and_fastest_frequency():
    """Page values: the fastest frequency's angle equals the position in
    radians, and cos(200000) has magnitude ~0.997 (the fp32 device value 0.0
    was off by 0.997) -- gaudi-cookbook 'The RoPE fix for large positions'."""
    g = json.load(open(GOLDEN))
    f = oracle.inv_freq(1e4, g["partial_rotary_dims"]["value"])
    assert f[0] == g["fastest_frequency_rad_per_position"]["value"]
    e = np.zeros((1, 1, 192))
    e[0, 0, 0] = 1.0
    y = oracle.rope(e, [200000], 1e4)
    assert round(abs(y[0, 0, 0]), 3) == g["cos_200000_magnitude"]["value_approx"]
    # the pair rotates by +angle: e_0 -> (cos a, sin a) in dims (0, 32)
    y1 = oracle.rope(e, [1], 1e4)
    assert abs(y1[0, 0, 0] - math.cos(1.0)) < 1e-15 and abs(y1[0, 0, 32] - math.sin(1.0)) < 1e-15


# ------------------------------------------------------------- P9 GQA
def test_p9_gqa_grouping_equals_explicit_repeat():
    r = rng(9)
    T = 140
    q, k, v = r.standard_normal((T, 8, 192)), r.standard_normal((T, 2, 192)), r.standard_normal((T, 2, 128))
    s = 1 + 0.25 * r.standard_normal(8)
    pos = np.arange(T)
    og = oracle.attn_linear(q, pos, k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    om = oracle.attn_linear(q, pos, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0,
                            window=128, tau=TAU, lam=LAM, sinks=s)
    assert np.array_equal(og, om)


# ----------------------------------------------------- P11 value scale
def test_p11_value_scale_before_equals_after():
    """colibri 'What the engine implements': values are multiplied by the
    value scale before attention; by linearity this equals scaling after."""
    r = rng(11)
    T = 100
    q, k, v = r.standard_normal((T, 4, 192)), r.standard_normal((T, 1, 192)), r.standard_normal((T, 1, 128))
    s = 1 + 0.25 * r.standard_normal(4)
    pos = np.arange(T)
    before = oracle.attn_linear(q, pos, k, v * LAM, 0, window=128, tau=TAU, lam=1.0, sinks=s)
    inside = oracle.attn_linear(q, pos, k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    after = oracle.attn_linear(q, pos, k, v, 0, window=128, tau=TAU, lam=1.0, sinks=s) * LAM
    assert np.array_equal(before, inside)
    assert rel(after, inside) < 1e-15


# ------------------------------------------------ P12 / P13 closed forms
def test_p12_window_one_closed_form():
    """W = 1: o_i = lam * v_i * sigmoid(l_ii - sigma)."""
    r = rng(12)
    T = 20
    q, k, v = r.standard_normal((T, 4, 192)), r.standard_normal((T, 2, 192)), r.standard_normal((T, 2, 128))
    s = 1 + 0.25 * r.standard_normal(4)
    o = oracle.attn_linear(q, np.arange(T), k, v, 0, window=1, tau=TAU, lam=LAM, sinks=s)
    g = np.array([0, 0, 1, 1])
    lii = TAU * np.einsum("thd,thd->th", q, k[:, g, :])
    expect = LAM * v[:, g, :] / (1.0 + np.exp(s[None, :] - lii))[..., None]
    assert rel(o, expect) < 1e-13


def test_p13_zero_query_closed_form():
    """q = 0 makes every logit 0: o = lam * sum_{j in J} v_j / (|J| + e^sigma)."""
    r = rng(13)
    T = 300
    k, v = r.standard_normal((T, 1, 192)), r.standard_normal((T, 1, 128))
    q = np.zeros((T, 4, 192))
    s = 1 + 0.25 * r.standard_normal(4)
    o = oracle.attn_linear(q, np.arange(T), k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    for i in (0, 1, 126, 127, 128, 299):
        lo = max(0, i - 127)
        n = i - lo + 1
        expect = LAM * v[lo:i + 1, 0, :].sum(0)[None, :] / (n + np.exp(s))[:, None]
        assert rel(o[i], expect) < 1e-13


# -------------------------------------------- P14 decode = prefill row
def test_p14_decode_equals_prefill_row_and_batch_independence():
    """colibri 'Correctness' / 'System One mode': prefill in blocks of 1 and 3
    gives the same bytes; a row depends only on its own inputs.  A decode at
    position P equals prefill row P, bitwise, and the ring decode agrees."""
    r = rng(14)
    T = 260
    q, k, v = r.standard_normal((T, 8, 192)), r.standard_normal((T, 2, 192)), r.standard_normal((T, 2, 128))
    s = 1 + 0.25 * r.standard_normal(8)
    pos = np.arange(T)
    full = oracle.attn_linear(q, pos, k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    perm = r.permutation(T)
    shuffled = oracle.attn_linear(q[perm], pos[perm], k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
    assert np.array_equal(shuffled, full[perm])
    for P in (0, 5, 127, 128, 259):
        one = oracle.attn_linear(q[P:P + 1], [P], k, v, 0, window=128, tau=TAU, lam=LAM, sinks=s)
        assert np.array_equal(one[0], full[P])
        kring = np.zeros((1, 2, 128, 192))
        vring = np.zeros((1, 2, 128, 128))
        for p in range(P + 1):
            kring[0, :, p % 128] = k[p]
            vring[0, :, p % 128] = v[p]
        od = oracle.ring_decode(q[P:P + 1], [P], kring, vring, tau=TAU, lam=LAM, sinks=s)
        assert rel(od[0], full[P]) < 1e-13
