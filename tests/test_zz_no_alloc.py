"""hsw_full_decode_splitk_noalloc (the split-K full decode with its partials
in the library's scratch array, for callers that cannot allocate) against
hsw_full_decode_splitk with a caller workspace, through the C ABI: two calls
in a row, the second smaller (the scratch keeps the first call's contents),
each bit for bit equal to the workspace call and within the parity bar of
the fp64 oracle; a call whose partials exceed the scratch is refused before
any launch."""
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


def both_calls(batch, chunk, sinks):
    """RoPE of the new tokens into the pool, then the workspace call and the
    no-allocation call on the same q_rot and pool."""
    shape = batch["shape"]
    S = batch["ctx_len"].shape[0]
    kpool, vpool = batch["kpool"].to(DEV), batch["vpool"].to(DEV)
    rows = kpool.shape[0]
    q_rot = torch.empty((S, shape.n_q_heads, 192), dtype=torch.bfloat16, device=DEV)
    hsw.hsw_rope_partial_kv_write(shape, S, batch["q"].to(DEV), batch["k"].to(DEV), batch["v"].to(DEV),
                                  batch["pos"].to(DEV), batch["seq"].to(DEV), hsw.HSW_DST_POOL, kpool, vpool, rows,
                                  batch["seq_base"].to(DEV), q_rot)
    max_ctx = int(batch["ctx_len"].max())
    ctx, base = batch["ctx_len"].to(DEV), batch["seq_base"].to(DEV)
    d_sinks = None if sinks is None else sinks.to(DEV)
    wsb = hsw.hsw_full_decode_workspace_bytes(shape, S, max_ctx, chunk)
    assert wsb <= hsw.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=DEV)
    out_ws = torch.full((S, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    hsw.hsw_full_decode_splitk(shape, S, max_ctx, ctx, base, q_rot, kpool, vpool, rows, d_sinks, chunk, ws, wsb,
                               out_ws)
    out_na = torch.full_like(out_ws, SENTINEL)
    hsw.hsw_full_decode_splitk_noalloc(shape, S, max_ctx, ctx, base, q_rot, kpool, vpool, rows, d_sinks, chunk,
                                       out_na)
    torch.cuda.synchronize()
    return q_rot, kpool, vpool, out_ws, out_na


def oracle_rows(batch, q_rot, kpool, vpool, sinks):
    shape = batch["shape"]
    L, base = batch["ctx_len"].tolist(), batch["seq_base"].tolist()
    qr = f64(q_rot)
    return np.stack([oracle.attn_linear(qr[s:s + 1], [L[s] - 1], f64(kpool[base[s]:base[s] + L[s]]),
                                        f64(vpool[base[s]:base[s] + L[s]]), 0, window=0,
                                        sinks=None if sinks is None else f64(sinks), **shape_kw(shape))[0]
                     for s in range(len(L))])


def test_noalloc_full_decode_equals_workspace_call_twice():
    note("noalloc full decode: first call, 12 sequences up to 40000 keys, chunk 2048")
    first = wl.full_decode_batch(seed=111, n_seqs=12, len_lo=1, len_hi=40000)
    q_rot, kp, vp, out_ws, out_na = both_calls(first, 2048, None)
    assert torch.equal(out_na, out_ws), "no-allocation call differs from the workspace call"
    ma, mr = assert_close(f64(out_na), oracle_rows(first, q_rot, kp, vp, None), what="noalloc first call")
    print(f"noalloc first call: bitwise equal; max_abs={ma:.2e} mean_rel={mr:.2e}")
    del kp, vp

    note("noalloc full decode: second, smaller call with sinks, chunk 1024")
    second = wl.full_decode_batch(seed=112, n_seqs=5, lengths=[1, 2048, 2049, 3000, 777], with_sinks=True)
    q_rot, kp, vp, out_ws, out_na = both_calls(second, 1024, second["sinks"])
    assert torch.equal(out_na, out_ws), "second no-allocation call differs (stale scratch?)"
    ma, mr = assert_close(f64(out_na), oracle_rows(second, q_rot, kp, vp, second["sinks"]),
                          what="noalloc second call")
    print(f"noalloc second call: bitwise equal; max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_noalloc_full_decode_refuses_partials_beyond_the_scratch():
    note("noalloc full decode: a request beyond the scratch")
    shape = wl.full_shape()
    S, max_ctx, chunk = 64, 131072, 2048            # 64 * 64 * 64 partials of 520 B: 136 MB
    assert hsw.hsw_full_decode_workspace_bytes(shape, S, max_ctx, chunk) > hsw.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.int64, device=DEV)
    out = torch.full((S, 64, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(hsw.HswError) as e:
        hsw.hsw_full_decode_splitk_noalloc(shape, S, max_ctx, t, t, out, out, out, 1, None, chunk, out)
    assert e.value.status == 5          # HSW_E_WORKSPACE, before any launch
    torch.cuda.synchronize()
    assert bool((out == SENTINEL).all())
