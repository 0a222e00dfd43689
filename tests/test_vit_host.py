"""Vision-encoder calls on the host (no GPU): the library's merge-unit
layout equals the oracle's exactly, and the ViT calls reject bad arguments
with the documented status before any launch (colibri "MiMo-V2.6 (Xiaomi)",
the "vision" entry: row and column order of the 2x2 merge units).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw",
                          reason="libhsw.so not built (python -m hybrid_sliding_window_amd.build)")
from hybrid_sliding_window_amd import workloads as wl  # noqa: E402

FAKE = 0x10000


@pytest.mark.parametrize("h,w", [(2, 2), (4, 4), (2, 6), (28, 36), (64, 64), (8, 130), (130, 8)])
def test_layout_equals_oracle(h, w):
    got = hsw.hsw_vit_layout(h, w)
    ref = oracle.vit_layout(h, w)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


def expect(status, fn, *args):
    with pytest.raises(hsw.HswError) as e:
        fn(*args)
    assert e.value.status == status, (e.value.status, status)


def test_layout_rejects_odd_or_empty_grids():
    for h, w in [(3, 4), (4, 5), (0, 4), (-2, 2)]:
        expect(2, hsw.hsw_vit_layout, h, w)


def test_vit_argument_errors():
    sh = hsw.make_shape(wl.vit_shape())
    full = hsw.make_shape(wl.vit_shape(window=0))
    args = (2, 100, FAKE, None, 1, FAKE, FAKE, FAKE, None, FAKE)
    hsw.hsw_vit_attention(sh, 0, 100, FAKE, None, 1, FAKE, FAKE, FAKE, None, FAKE)    # empty
    hsw.hsw_vit_attention(full, 2, 0, FAKE, None, 0, FAKE, FAKE, FAKE, None, FAKE)    # empty
    expect(1, hsw.hsw_vit_attention, sh, 2, 100, None, None, 1, FAKE, FAKE, FAKE, None, FAKE)
    expect(1, hsw.hsw_vit_attention, sh, 2, 100, FAKE, None, 1, FAKE, None, FAKE, None, FAKE)
    expect(3, hsw.hsw_vit_attention, sh, 2, 100, FAKE, None, 1, FAKE + 8, FAKE, FAKE, None, FAKE)
    expect(3, hsw.hsw_vit_attention, sh, 2, 100, FAKE, FAKE + 2, 1, FAKE, FAKE, FAKE, None, FAKE)
    w128 = hsw.make_shape(wl.vit_shape(window=128))
    expect(2, hsw.hsw_vit_attention, w128, *args)
    g3 = hsw.make_shape(wl.vit_shape(hq=12, hkv=4))
    expect(2, hsw.hsw_vit_attention, g3, *args)
    d128 = hsw.make_shape(wl.vit_shape())
    d128.d_qk = d128.d_v = d128.rope_dim = 128
    expect(2, hsw.hsw_vit_attention, d128, *args)
    vs = hsw.make_shape(wl.vit_shape())
    vs.value_scale = 0.7
    expect(2, hsw.hsw_vit_attention, vs, *args)
    f32 = hsw.make_shape(wl.vit_shape())
    f32.dtype = f32.out_dtype = hsw.HSW_F32
    expect(2, hsw.hsw_vit_attention, f32, *args)
    expect(2, hsw.hsw_vit_attention, sh, -1, 100, FAKE, None, 1, FAKE, FAKE, FAKE, None, FAKE)


def test_vit_rope_argument_errors():
    sh = hsw.make_shape(wl.vit_shape())
    hsw.hsw_vit_rope_2d(sh, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)                     # empty
    expect(1, hsw.hsw_vit_rope_2d, sh, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE)        # q without q_out
    expect(1, hsw.hsw_vit_rope_2d, sh, 4, None, None, FAKE, FAKE, None, None)        # nothing to rotate
    expect(1, hsw.hsw_vit_rope_2d, sh, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE)        # no rows
    expect(3, hsw.hsw_vit_rope_2d, sh, 4, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE)
    part = hsw.make_shape(wl.vit_shape())
    part.rope_dim = 32
    expect(2, hsw.hsw_vit_rope_2d, part, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    f32 = hsw.make_shape(wl.vit_shape())
    f32.dtype = hsw.HSW_F32
    expect(4, hsw.hsw_vit_rope_2d, f32, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
