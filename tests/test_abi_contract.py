"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/hsw.h declares, rejects bad arguments on the host with the
documented status (launching nothing), treats empty calls as no-ops, and its
host-side layout arithmetic reproduces byte counts the pages print.
"""
from __future__ import annotations

import ctypes
import json
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsw.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_values.json")

hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw",
                          reason="libhsw.so not built (python -m hybrid_sliding_window_amd.build)")
from hybrid_sliding_window_amd import workloads as wl  # noqa: E402

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails or is empty


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(hsw_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", hsw.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hsw_[a-z0-9_]+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(hsw.lib, n)
    assert set(hsw.EXPORTED) == set(names)


def test_status_strings():
    for code in range(7):
        assert hsw.lib.hsw_status_str(code).decode().startswith(hsw.STATUS[code])
    assert "gfx950" in hsw.hsw_version()


def swa():
    return hsw.make_shape(wl.swa_shape())


def full():
    return hsw.make_shape(wl.full_shape())


def expect(status, fn, *args, **kw):
    with pytest.raises(hsw.HswError) as e:
        fn(*args, **kw)
    assert e.value.status == status, str(e.value)


def test_rope_argument_errors():
    sh = swa()
    args = dict(n_tokens=4, q=FAKE, k=FAKE, v=FAKE, pos=FAKE, seq=FAKE, dst_kind=hsw.HSW_DST_RING,
                k_dst=FAKE, v_dst=FAKE, dst_capacity=4, seq_base=None, q_rot=FAKE)
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "q": None})
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "seq": None})
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "dst_kind": hsw.HSW_DST_POOL})  # no seq_base
    expect(3, hsw.hsw_rope_partial_kv_write, sh, **{**args, "k": FAKE + 2})
    expect(2, hsw.hsw_rope_partial_kv_write, sh, **{**args, "dst_kind": 7})
    expect(2, hsw.hsw_rope_partial_kv_write, sh, **{**args, "n_tokens": -1})
    bad = swa()
    bad.rope_dim = 24
    expect(2, hsw.hsw_rope_partial_kv_write, bad, **args)
    bad = swa()
    bad.n_kv_heads = 3
    expect(2, hsw.hsw_rope_partial_kv_write, bad, **args)
    bad = swa()
    bad.dtype = 9
    expect(4, hsw.hsw_rope_partial_kv_write, bad, **args)
    ring_full = full()
    expect(2, hsw.hsw_rope_partial_kv_write, ring_full, **args)  # ring needs a window
    # empty call: nothing launched, nothing touched
    hsw.hsw_rope_partial_kv_write(sh, **{**args, "n_tokens": 0})


def test_rope_k_only_staging_contract():
    """v and v_dst both NULL is the K-only staging write; anything else
    without V is refused before a launch."""
    sh = swa()
    args = dict(n_tokens=4, q=None, k=FAKE, v=None, pos=FAKE, seq=None, dst_kind=hsw.HSW_DST_STAGING,
                k_dst=FAKE, v_dst=None, dst_capacity=4, seq_base=None, q_rot=None)
    hsw.hsw_rope_partial_kv_write(sh, **{**args, "n_tokens": 0})  # accepted (empty: no launch)
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "v_dst": FAKE})  # v missing alone
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "v": FAKE})      # v_dst missing alone
    for kind in (hsw.HSW_DST_RING, hsw.HSW_DST_POOL):                       # caches always take V
        expect(1, hsw.hsw_rope_partial_kv_write, sh,
               **{**args, "dst_kind": kind, "seq": FAKE, "seq_base": FAKE})


def test_vit_window_attention_rope_argument_errors():
    """Window 64 only (full blocks rotate once with the 2D RoPE call), the
    coordinates required, nothing launched on an error or an empty call."""
    sh = wl.vit_shape(16, 4, 64)
    args = (1, 64, FAKE, None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    hsw.hsw_vit_window_attention_rope(sh, 0, 64, FAKE, None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)  # empty
    expect(2, hsw.hsw_vit_window_attention_rope, wl.vit_shape(16, 4, 0), *args)           # full block
    expect(1, hsw.hsw_vit_window_attention_rope, sh, 1, 64, FAKE, None, 1, None, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(1, hsw.hsw_vit_window_attention_rope, sh, 1, 64, FAKE, None, 1, FAKE, None, FAKE, FAKE, FAKE, None, FAKE)
    expect(3, hsw.hsw_vit_window_attention_rope, sh, 1, 64, FAKE, None, 1, FAKE + 2, FAKE, FAKE, FAKE, FAKE, None,
           FAKE)                                                                               # row misaligned


def test_attention_argument_errors():
    sh, fs = swa(), full()
    expect(2, hsw.hsw_swa_prefill, fs, 1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(1, hsw.hsw_swa_prefill, sh, 1, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(3, hsw.hsw_swa_prefill, sh, 1, 8, FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    hsw.hsw_swa_prefill(sh, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(2, hsw.hsw_swa_decode, fs, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(1, hsw.hsw_swa_decode, sh, 2, FAKE, FAKE, None, FAKE, None, FAKE)
    hsw.hsw_swa_decode(sh, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    need = hsw.hsw_full_decode_workspace_bytes(fs, 4, 10000, 2048)
    assert need > 0
    expect(5, hsw.hsw_full_decode_splitk, fs, 4, 10000, FAKE, FAKE, FAKE, FAKE, FAKE, 40000, None,
           2048, FAKE, need - 16, FAKE)
    expect(2, hsw.hsw_full_decode_splitk, fs, 4, 10000, FAKE, FAKE, FAKE, FAKE, FAKE, 40000, None,
           100, FAKE, need, FAKE)
    expect(2, hsw.hsw_full_decode_splitk, sh, 4, 10000, FAKE, FAKE, FAKE, FAKE, FAKE, 40000, None,
           2048, FAKE, need, FAKE)
    expect(2, hsw.hsw_full_prefill_chunk, sh, 1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None, FAKE)
    expect(1, hsw.hsw_full_prefill_chunk, fs, 1, 8, FAKE, FAKE, None, FAKE, FAKE, FAKE, 100, None, FAKE)
    hsw.hsw_full_prefill_chunk(fs, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None, FAKE)


def test_fused_qrope_argument_errors():
    """The calls that rotate q themselves: shapes outside their kernels and
    missing pointers are rejected on the host; K/V-only RoPE takes q and
    q_rot both NULL, not one of them."""
    sh, fs = swa(), full()
    pre = (1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    hsw.hsw_swa_prefill_qrope(sh, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)  # empty
    expect(2, hsw.hsw_swa_prefill_qrope, fs, *pre)
    expect(1, hsw.hsw_swa_prefill_qrope, sh, 1, 8, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(3, hsw.hsw_swa_prefill_qrope, sh, 1, 8, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    mha = hsw.make_shape(wl.swa_shape(8, 8))          # one q head per KV head: no prefill table
    expect(2, hsw.hsw_swa_prefill_qrope, mha, *pre)
    r32 = swa()
    r32.rope_dim = 32
    expect(2, hsw.hsw_swa_prefill_qrope, r32, *pre)
    expect(2, hsw.hsw_swa_decode_qrope, r32, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    f32 = hsw.make_shape(wl.swa_shape(dtype=__import__("torch").float32))
    expect(2, hsw.hsw_swa_prefill_qrope, f32, *pre)
    expect(2, hsw.hsw_swa_decode_qrope, f32, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    expect(1, hsw.hsw_swa_decode_qrope, sh, 2, FAKE, None, FAKE, FAKE, None, FAKE)
    expect(2, hsw.hsw_swa_decode_qrope, fs, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    hsw.hsw_swa_decode_qrope(sh, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    hsw.hsw_swa_decode_qrope(mha, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE)   # G = 1 decode is supported
    # the full-attention calls that rotate q themselves
    fpre = (1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None, FAKE)
    hsw.hsw_full_prefill_chunk_qrope(fs, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None, FAKE)  # empty
    expect(1, hsw.hsw_full_prefill_chunk_qrope, fs, 1, 8, FAKE, FAKE, FAKE, None, FAKE, FAKE, 100, None, FAKE)
    expect(3, hsw.hsw_full_prefill_chunk_qrope, fs, 1, 8, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 100, None, FAKE)
    fmha = hsw.make_shape(wl.full_shape(4, 4))        # one q head per KV head: no prefill table
    expect(2, hsw.hsw_full_prefill_chunk_qrope, fmha, *fpre)
    fr32 = full()
    fr32.rope_dim = 32
    expect(2, hsw.hsw_full_prefill_chunk_qrope, fr32, *fpre)
    ff32 = hsw.make_shape(wl.full_shape(dtype=__import__("torch").float32))
    expect(2, hsw.hsw_full_prefill_chunk_qrope, ff32, *fpre)
    need = hsw.hsw_full_decode_workspace_bytes(fs, 4, 10000, 2048)
    dec = (4, 10000, FAKE, FAKE, FAKE, FAKE, FAKE, 40000, None, 2048, FAKE, need, FAKE)
    expect(2, hsw.hsw_full_decode_splitk_qrope, fr32, *dec)
    expect(2, hsw.hsw_full_decode_splitk_qrope, ff32, *dec)
    expect(1, hsw.hsw_full_decode_splitk_qrope, fs, 4, 10000, FAKE, FAKE, None, FAKE, FAKE, 40000, None,
           2048, FAKE, need, FAKE)
    expect(5, hsw.hsw_full_decode_splitk_qrope, fs, 4, 10000, FAKE, FAKE, FAKE, FAKE, FAKE, 40000, None,
           2048, FAKE, need - 16, FAKE)
    hsw.hsw_full_decode_splitk_qrope(fs, 0, 10000, FAKE, FAKE, FAKE, FAKE, FAKE, 40000, None, 2048, FAKE, 0, FAKE)
    hsw.hsw_full_decode_splitk_qrope(fmha, 0, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 400, None, 2048, FAKE, 0,
                                     FAKE)  # G = 1 decode is supported
    args = dict(n_tokens=0, q=None, k=FAKE, v=FAKE, pos=FAKE, seq=FAKE, dst_kind=hsw.HSW_DST_RING,
                k_dst=FAKE, v_dst=FAKE, dst_capacity=4, seq_base=None, q_rot=None)
    hsw.hsw_rope_partial_kv_write(sh, **args)                              # K/V only, empty
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "q_rot": FAKE})
    expect(1, hsw.hsw_rope_partial_kv_write, sh, **{**args, "q": FAKE})


def test_workspace_size_formula():
    fs = full()
    for S, L, C in [(64, 131072, 2048), (3, 1, 2048), (1, 4097, 1024)]:
        nc = math.ceil(L / C)
        ml = (2 * S * 64 * nc + 3) // 4 * 4
        assert hsw.hsw_full_decode_workspace_bytes(fs, S, L, C) == 4 * (ml + S * 64 * nc * 128)


def test_p10_kv_bytes_reproduce_page_values():
    """Layout arithmetic against byte counts the pages print (golden file)."""
    g = json.load(open(GOLDEN))
    RING, POOL = hsw.HSW_DST_RING, hsw.HSW_DST_POOL
    # 9 full layers, TP8 -> 1 KV head per card, V zero-padded to 192, bf16
    assert hsw.hsw_kv_bytes(POOL, 1, 1, 0, 1, 192, 192, 2, 9) == g["full_kv_bytes_per_token_per_card_windowed_kv"]["value"]
    # stock: all 48 layers keep full-length KV
    assert hsw.hsw_kv_bytes(POOL, 1, 1, 0, 1, 192, 192, 2, 48) == g["full_kv_bytes_per_token_per_card_stock"]["value"]
    # colibri snapshot: 39 rings x 128 slots x 8 heads x (192+128) f32 ~ 50 MB, whatever the context
    snap = hsw.hsw_kv_bytes(RING, 1, 123456, 128, 8, 192, 128, 4, 39)
    assert snap == hsw.hsw_kv_bytes(RING, 1, 7, 128, 8, 192, 128, 4, 39) == 51_118_080
    assert round(snap / 1e6, -1) == g["ring_snapshot_bytes_flash"]["value_approx_mb"]
    # Pro: 10 full layers x 8192 positions x 8 KV heads x (192+128) f32 = 0.78 GiB
    pro = hsw.hsw_kv_bytes(POOL, 1, 8192, 0, 8, 192, 128, 4, 10)
    assert round(pro / 2 ** 30, 2) == g["pro_full_kv_bytes_8k"]["value_gib_approx"]
    assert hsw.hsw_kv_bytes(7, 1, 1, 0, 1, 1, 1, 1, 1) == -1
    assert hsw.hsw_kv_bytes(RING, 1, 1, 0, 1, 1, 1, 1, 1) == -1
