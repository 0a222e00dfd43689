"""The checked build (libhsw_checked.so, HSW_CHECK_DEVICE=1) on the GPU.

On valid inputs every call of the checked build writes exactly the bytes the
release build writes (its kernels differ only by a test of the check flag at
their start), and the flag stays clear.  Out-of-contract device values --
each chosen so that the release kernels stay inside their buffers too (a
negative decode position, a context length past max_ctx, a ring sequence
outside the ring, a prefill reaching past the pool) -- are reported with the
rule's code and the offending element, the call writes nothing, and the next
call runs again once the flag was read.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, f64, note, shape_kw
from parity import assert_close

pytestmark = pytest.mark.gpu

hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw")
from hybrid_sliding_window_amd import workloads as wl  # noqa: E402

SENTINEL = -7.25
RING, POOL, STAGING = hsw.HSW_DST_RING, hsw.HSW_DST_POOL, hsw.HSW_DST_STAGING
POSITION, CU_SEQLENS, POOL_RANGE, RING_SEQ, CTX_LEN = 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def chk():
    m = hsw.load_library(hsw.CHECKED_LIB_PATH)
    assert m.hsw_device_checks_enabled()
    assert m.hsw_device_check_status() == (0, 0, -1), "flag not clear at start"
    return m


def d(t):
    return None if t is None else t.to(DEV)


def decode_run(m, batch, pos=None):
    """RoPE of the new tokens into the rings, then the windowed decode."""
    shape = batch["shape"]
    S = batch["pos"].shape[0]
    pos = d(batch["pos"] if pos is None else pos)
    kring, vring = d(batch["kring"]), d(batch["vring"])
    q_rot = torch.empty_like(d(batch["q"]))
    m.hsw_rope_partial_kv_write(shape, S, d(batch["q"]), d(batch["k"]), d(batch["v"]), d(batch["pos"]),
                                d(batch["seq"]), RING, kring, vring, S, None, q_rot)
    out = torch.full((S, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    m.hsw_swa_decode(shape, S, pos, q_rot, kring, vring, d(batch["sinks"]), out)
    torch.cuda.synchronize()
    return q_rot, kring, vring, out


def prefill_run(m, batch):
    shape = batch["shape"]
    T = batch["q"].shape[0]
    S = batch["start_pos"].shape[0]
    lens = batch["cu_seqlens"][1:] - batch["cu_seqlens"][:-1]
    q_rot = torch.empty_like(d(batch["q"]))
    kst, vst = torch.empty_like(d(batch["k"])), torch.empty_like(d(batch["v"]))
    m.hsw_rope_partial_kv_write(shape, T, d(batch["q"]), d(batch["k"]), d(batch["v"]), d(batch["pos"]), None,
                                STAGING, kst, vst, T, None, q_rot)
    kring, vring = d(batch["kring"]), d(batch["vring"])
    out = torch.full((T, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    m.hsw_swa_prefill(shape, S, int(lens.max()), d(batch["cu_seqlens"]), d(batch["start_pos"]), q_rot, kst, vst,
                      kring, vring, d(batch["sinks"]), out)
    torch.cuda.synchronize()
    return kring, vring, out


def full_decode_run(m, batch, max_ctx=None, chunk=1024):
    shape = batch["shape"]
    S = batch["ctx_len"].shape[0]
    kpool, vpool = d(batch["kpool"]), d(batch["vpool"])
    rows = kpool.shape[0]
    q_rot = torch.empty_like(d(batch["q"]))
    m.hsw_rope_partial_kv_write(shape, S, d(batch["q"]), d(batch["k"]), d(batch["v"]), d(batch["pos"]),
                                d(batch["seq"]), POOL, kpool, vpool, rows, d(batch["seq_base"]), q_rot)
    max_ctx = int(batch["ctx_len"].max()) if max_ctx is None else max_ctx
    wsb = hsw.hsw_full_decode_workspace_bytes(shape, S, max_ctx, chunk)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=DEV)
    out = torch.full((S, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    m.hsw_full_decode_splitk(shape, S, max_ctx, d(batch["ctx_len"]), d(batch["seq_base"]), q_rot, kpool, vpool,
                             rows, None, chunk, ws, wsb, out)
    torch.cuda.synchronize()
    return q_rot, kpool, vpool, out


def full_prefill_run(m, batch, start_pos=None):
    shape = batch["shape"]
    T = batch["q"].shape[0]
    S = batch["start_pos"].shape[0]
    kpool, vpool = d(batch["kpool"]), d(batch["vpool"])
    rows = kpool.shape[0]
    q_rot = torch.empty_like(d(batch["q"]))
    m.hsw_rope_partial_kv_write(shape, T, d(batch["q"]), d(batch["k"]), d(batch["v"]), d(batch["pos"]),
                                d(batch["seq"]), POOL, kpool, vpool, rows, d(batch["seq_base"]), q_rot)
    lens = batch["cu_seqlens"][1:] - batch["cu_seqlens"][:-1]
    out = torch.full((T, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    st = batch["start_pos"] if start_pos is None else start_pos
    m.hsw_full_prefill_chunk(shape, S, int(lens.max()), d(batch["cu_seqlens"]), d(st), d(batch["seq_base"]),
                             q_rot, kpool, vpool, rows, None, out)
    torch.cuda.synchronize()
    return out


def test_checked_build_equals_release_build_on_valid_inputs(chk):
    note("checked build: windowed decode at positions up to 2^33")
    positions = [0, 1, 127, 128, 524288, 2 ** 31 - 1, 2 ** 31 + 5, 2 ** 33 + 77]
    b = wl.swa_decode_batch(seed=101, n_seqs=len(positions), positions=positions)
    r = decode_run(hsw, b)
    c = decode_run(chk, b)
    assert chk.hsw_device_check_status() == (0, 0, -1)
    for x, y in zip(r, c):
        assert torch.equal(x, y)
    ref = oracle.ring_decode(f64(r[0]), b["pos"].numpy(), f64(r[1]), f64(r[2]), sinks=f64(b["sinks"]),
                             **shape_kw(b["shape"]))
    assert_close(f64(c[3]), ref, what="checked windowed decode")

    note("checked build: windowed prefill, ragged, starts up to 2^32")
    b = wl.swa_prefill_batch(seed=102, n_seqs=3, seqlens=(200, 0, 77), start_pos=(0, 9, 2 ** 32 + 3))
    for x, y in zip(prefill_run(hsw, b), prefill_run(chk, b)):
        assert torch.equal(x, y)
    assert chk.hsw_device_check_status() == (0, 0, -1)

    note("checked build: full decode and full prefill")
    b = wl.full_decode_batch(seed=103, n_seqs=3, lengths=[1, 300, 2500])
    for x, y in zip(full_decode_run(hsw, b), full_decode_run(chk, b)):
        assert torch.equal(x, y)
    b = wl.full_prefill_batch(seed=104, n_seqs=2, seqlens=(70, 1), start_pos=(200, 0))
    assert torch.equal(full_prefill_run(hsw, b), full_prefill_run(chk, b))
    assert chk.hsw_device_check_status() == (0, 0, -1)


def test_checked_build_flags_contract_violations_and_writes_nothing(chk):
    note("checked build: a negative decode position")
    b = wl.swa_decode_batch(seed=105, n_seqs=6, positions=[3, 200, 7, 9, 11, 500])
    bad = b["pos"].clone()
    bad[4] = -5
    *_, out = decode_run(chk, b, pos=bad)
    assert chk.hsw_device_check_status() == (9, POSITION, 4)
    assert bool((out == SENTINEL).all()), "the checked decode wrote despite the violation"
    assert chk.hsw_device_check_status() == (0, 0, -1), "the flag was not cleared"

    note("checked build: a ring sequence outside the ring")
    shape = b["shape"]
    seq = b["seq"].clone()
    seq[2] = 6                                    # the ring holds sequences 0..5
    kring, vring = d(b["kring"]), d(b["vring"])
    kr0 = kring.clone()
    q_rot = torch.full_like(d(b["q"]), SENTINEL)
    chk.hsw_rope_partial_kv_write(shape, 6, d(b["q"]), d(b["k"]), d(b["v"]), d(b["pos"]), d(seq), RING, kring,
                                  vring, 6, None, q_rot)
    assert chk.hsw_device_check_status() == (9, RING_SEQ, 2)
    assert torch.equal(kring, kr0) and bool((q_rot == SENTINEL).all())

    note("checked build: a context length past max_ctx")
    b = wl.full_decode_batch(seed=106, n_seqs=3, lengths=[10, 300, 40])
    *_, out = full_decode_run(chk, b, max_ctx=299)
    assert chk.hsw_device_check_status() == (9, CTX_LEN, 1)
    assert bool((out == SENTINEL).all())

    note("checked build: a prefill chunk reaching past the pool")
    b = wl.full_prefill_batch(seed=107, n_seqs=2, seqlens=(30, 20), start_pos=(40, 10))
    st = b["start_pos"].clone()
    st[1] = 11                                     # rows base + 11 .. base + 30: one past the pool
    out = full_prefill_run(chk, b, start_pos=st)
    code = chk.hsw_device_check_status()
    assert code == (9, POOL_RANGE, 1)
    assert bool((out == SENTINEL).all())

    note("checked build: a valid call after the violations")
    b = wl.swa_decode_batch(seed=108, n_seqs=4, positions=[0, 50, 128, 9999])
    assert torch.equal(decode_run(chk, b)[3], decode_run(hsw, b)[3])
    assert chk.hsw_device_check_status() == (0, 0, -1)
