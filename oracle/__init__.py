"""fp64 CPU oracle for the hybrid sliding-window attention core.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library (``hybrid_sliding_window_amd``) and never imports it.

The arithmetic lives in ``hsw_oracle.c`` (plain loops in double precision);
this module builds it with gcc on demand and wraps each function for numpy
float64 / int64 arrays.  Every wrapper states the passage of the pages it
follows; see the C file for the definitions.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, a library routine, an independent
brute force and values the pages print), except the softmax scale, which the
pages never state: it is an argument (1/sqrt(192) by the plainest reading) and
is "parity unpinned" as a constant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hsw_oracle.c")
_LIB = os.path.join(_HERE, "libhsw_oracle.so")
_lock = threading.Lock()
_lib = None

RING, POOL, STAGING = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile hsw_oracle.c into libhsw_oracle.so with gcc (IEEE fp64, no
    fast-math, no FMA contraction so every product rounds once as written;
    -O3 vectorises only loops whose lanes are independent sums, so no sum is
    reordered)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.hswo_num_threads.restype = i32
            lib.hswo_inv_freq.argtypes = [f64, i32, P]
            lib.hswo_rope.argtypes = [i64, i32, i32, i32, f64, P, P, P]
            lib.hswo_dst_index.argtypes = [i32, i64, i64, i64, i64]
            lib.hswo_dst_index.restype = i64
            lib.hswo_attn_linear.argtypes = [i32, i32, i32, i32, i64, f64, f64, P,
                                             i64, P, P, i64, P, P, i64, P, P]
            lib.hswo_attn_linear.restype = i32
            lib.hswo_ring_decode.argtypes = [i32, i32, i32, i32, i64, f64, f64, P,
                                             i64, P, P, P, P, P, P]
            lib.hswo_ring_decode.restype = i32
            lib.hswo_attn_partial.argtypes = [i32, i32, i32, i32, i64, f64, f64,
                                              i64, P, P, i64, P, P, i64, i64, i64,
                                              P, P, P]
            lib.hswo_attn_partial.restype = i32
            lib.hswo_join_sink.argtypes = [i64, i32, P, P, P, P]
            lib.hswo_lse_merge.argtypes = [i64, i64, i32, P, P, P, P, P]
            lib.hswo_vit_layout.argtypes = [i32, i32, P, P, P]
            lib.hswo_vit_layout.restype = i32
            lib.hswo_rope_2d.argtypes = [i64, i32, i32, f64, P, P, P, P]
            lib.hswo_vit_attn.argtypes = [i32, P, P, i32, i32, i32, i32, i32, i32, f64,
                                          P, P, P, P, P]
            lib.hswo_vit_attn.restype = i32
            _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().hswo_num_threads())


def inv_freq(theta: float, rope_dim: int) -> np.ndarray:
    """theta^(-2i/R) for i < R/2 (colibri, "What the engine implements")."""
    out = np.empty(rope_dim // 2, np.float64)
    _load().hswo_inv_freq(float(theta), int(rope_dim), _p(out))
    return out


def rope(x, pos, theta: float, rope_dim: int = 64) -> np.ndarray:
    """Partial rotate-half RoPE of x [T, H, D] at absolute positions pos [T]
    (colibri, "What the engine implements"; gaudi-cookbook, "The RoPE fix for
    large positions": angles in double precision)."""
    x = _f64(x)
    pos = _i64(pos)
    T, H, D = x.shape
    assert pos.shape == (T,)
    y = np.empty_like(x)
    _load().hswo_rope(T, H, D, int(rope_dim), float(theta), _p(pos), _p(x), _p(y))
    return y


def dst_index(kind: int, t: int, pos: int, seq_base: int = 0, ring_slots: int = 128) -> int:
    """Ring slot pos mod 128 / pool row seq_base + pos / staging row t
    (colibri, "System One mode and prompt reuse")."""
    return int(_load().hswo_dst_index(int(kind), int(t), int(pos), int(seq_base), int(ring_slots)))


def attn_linear(q, qpos, k, v, kpos0: int, *, window: int, tau: float, lam: float,
                sinks=None, want_lse: bool = False):
    """Attention of queries q [nq, Hq, Dqk] at positions qpos over K/V
    [nk, Hkv, D] holding positions kpos0 .. kpos0+nk-1 (window 0 = full
    causal).  colibri "What the engine implements"; gaudi-cookbook "What was
    built" (exactly the last 128 positions)."""
    q, k, v, qpos = _f64(q), _f64(k), _f64(v), _i64(qpos)
    nq, hq, dqk = q.shape
    nk, hkv, dqk2 = k.shape
    assert dqk2 == dqk and v.shape[:2] == (nk, hkv) and qpos.shape == (nq,)
    dv = v.shape[2]
    s = None if sinks is None else _f64(sinks)
    o = np.empty((nq, hq, dv), np.float64)
    lse = np.empty((nq, hq), np.float64)
    rc = _load().hswo_attn_linear(hq, hkv, dqk, dv, int(window), float(tau), float(lam),
                                  _p(s), nq, _p(q), _p(qpos), nk, _p(k), _p(v),
                                  int(kpos0), _p(o), _p(lse))
    if rc != 0:
        raise ValueError("oracle attn_linear: rc=%d (a needed key is missing)" % rc)
    return (o, lse) if want_lse else o


def ring_decode(q, pos, kring, vring, *, tau: float, lam: float, sinks=None,
                want_lse: bool = False):
    """Decode q [S, Hq, Dqk] at positions pos [S] over rings [S, Hkv, W, D]
    where slot t holds position P - ((P - t) mod W), used iff >= 0
    (colibri "System One mode and prompt reuse")."""
    q, kring, vring, pos = _f64(q), _f64(kring), _f64(vring), _i64(pos)
    ns, hq, dqk = q.shape
    _, hkv, slots, _ = kring.shape
    dv = vring.shape[3]
    s = None if sinks is None else _f64(sinks)
    o = np.empty((ns, hq, dv), np.float64)
    lse = np.empty((ns, hq), np.float64)
    rc = _load().hswo_ring_decode(hq, hkv, dqk, dv, slots, float(tau), float(lam), _p(s),
                                  ns, _p(q), _p(pos), _p(kring), _p(vring), _p(o), _p(lse))
    if rc != 0:
        raise ValueError("oracle ring_decode: rc=%d" % rc)
    return (o, lse) if want_lse else o


def attn_partial(q, qpos, k, v, kpos0: int, a: int, b: int, *, window: int, tau: float,
                 lam: float):
    """Unnormalised split-K partial (m, l, acc) over key positions [a, b)."""
    q, k, v, qpos = _f64(q), _f64(k), _f64(v), _i64(qpos)
    nq, hq, dqk = q.shape
    nk, hkv, _ = k.shape
    dv = v.shape[2]
    m = np.empty((nq, hq), np.float64)
    l = np.empty((nq, hq), np.float64)
    acc = np.empty((nq, hq, dv), np.float64)
    rc = _load().hswo_attn_partial(hq, hkv, dqk, dv, int(window), float(tau), float(lam),
                                   nq, _p(q), _p(qpos), nk, _p(k), _p(v), int(kpos0),
                                   int(a), int(b), _p(m), _p(l), _p(acc))
    if rc != 0:
        raise ValueError("oracle attn_partial: rc=%d" % rc)
    return m, l, acc


def join_sink(m, l, acc, sink):
    """Fold a sink logit into partials (denominator only); returns new arrays."""
    m, l, acc = _f64(m).copy(), _f64(l).copy(), _f64(acc).copy()
    sink = _f64(np.broadcast_to(sink, m.shape))
    n = m.size
    dv = acc.shape[-1]
    _load().hswo_join_sink(n, dv, _p(sink), _p(m), _p(l), _p(acc))
    return m, l, acc


def lse_merge(m, l, acc):
    """Log-sum-exp merge of partials stacked on axis 0: m, l [C, ...],
    acc [C, ..., Dv] -> (o [..., Dv], lse [...])."""
    m, l, acc = _f64(m), _f64(l), _f64(acc)
    C = m.shape[0]
    rest = m.shape[1:]
    n = int(np.prod(rest)) if rest else 1
    dv = acc.shape[-1]
    o = np.empty(rest + (dv,), np.float64)
    lse = np.empty(rest, np.float64)
    _load().hswo_lse_merge(C, n, dv, _p(m), _p(l), _p(acc), _p(o), _p(lse))
    return o, lse


# ---------------------------------------------------------------- vision (ViT)
def vit_layout(h: int, w: int):
    """(row [h*w], col [h*w], col_order [h*w]) int32 for an h x w patch grid
    in merge-unit order (colibri "MiMo-V2.6 (Xiaomi)", the "vision" entry:
    row and column order of the 2x2 merge units)."""
    n = h * w
    row, col, co = (np.empty(n, np.int32) for _ in range(3))
    rc = _load().hswo_vit_layout(int(h), int(w), _p(row), _p(col), _p(co))
    if rc != 0:
        raise ValueError("oracle vit_layout: h and w must be positive and even")
    return row, col, co


def rope_2d(x, row, col, theta: float = 1e4) -> np.ndarray:
    """2D rotate-half RoPE of x [T, H, D] at patch coordinates (row, col)
    (colibri, the "vision" entry: 2D RoPE)."""
    x = _f64(x)
    T, H, D = x.shape
    row = np.ascontiguousarray(row, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    assert row.shape == (T,) and col.shape == (T,)
    y = np.empty_like(x)
    _load().hswo_rope_2d(T, H, D, float(theta), _p(row), _p(col), _p(x), _p(y))
    return y


def vit_attn(q, k, v, cu, *, window: int, tau: float, order=None, sink_key: bool = False,
             sinks=None) -> np.ndarray:
    """ViT attention over pictures packed by cu (bidirectional; window 0 =
    the whole picture, else windows of `window` tokens in the order given,
    plus the picture's first token in that order as a sink key).  colibri
    "MiMo-V2.6 (Xiaomi)", the "vision" entry."""
    q, k, v, cu = _f64(q), _f64(k), _f64(v), _i64(cu)
    T, hq, d = q.shape
    _, hkv, _ = k.shape
    dv = v.shape[2]
    od = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    s = None if sinks is None else _f64(sinks)
    o = np.empty((T, hq, dv), np.float64)
    rc = _load().hswo_vit_attn(len(cu) - 1, _p(cu), _p(od), int(window), int(bool(sink_key)),
                               hq, hkv, d, dv, float(tau), _p(s), _p(q), _p(k), _p(v), _p(o))
    if rc != 0:
        raise ValueError("oracle vit_attn: rc=%d" % rc)
    return o
