"""GPU parity of the vision-encoder calls (hsw_vit_rope_2d,
hsw_vit_attention) against the fp64 oracle fed the exact tensors each call
consumed (colibri "MiMo-V2.6 (Xiaomi)", the "vision" entry: 2D RoPE, GQA,
full blocks and 64-token window blocks in alternating row / column order of
the 2x2 merge units; the window blocks add a sink placed at their leading
key).

Bars: rotated q/k within one bf16 ulp of the rounded fp64 value; attention
max_abs <= 2e-2 and mean_rel <= 2e-3.  The library's layout (coordinates
and column order) is checked equal to the oracle's on the CPU, so each side
uses its own.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, bf16_ulp, f64, note
from parity import assert_close, errors

pytestmark = pytest.mark.gpu

hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw")
from hybrid_sliding_window_amd import workloads as wl  # noqa: E402

SENTINEL = -7.25


def dev(t):
    return None if t is None else t.to(DEV)


def layouts(grids, lib):
    """Per-token row, col and the picture-local column order, concatenated."""
    rows, cols, orders = [], [], []
    for h, w in grids:
        r, c, o = hsw.hsw_vit_layout(h, w) if lib else oracle.vit_layout(h, w)
        rows.append(r)
        cols.append(c)
        orders.append(o)
    return np.concatenate(rows), np.concatenate(cols), np.concatenate(orders)


def run_attention(batch, shape, order=None, sink_key=True, q=None, k=None):
    T = batch["q"].shape[0]
    q = dev(batch["q"]) if q is None else q
    k = dev(batch["k"]) if k is None else k
    out = torch.full((T, shape.n_q_heads, 64), SENTINEL, dtype=torch.bfloat16, device=DEV)
    od = None if order is None else torch.from_numpy(order).to(DEV)
    hsw.hsw_vit_attention(shape, len(batch["lens"]), max(batch["lens"]), dev(batch["cu_seqlens"]), od,
                          int(sink_key), q, k, dev(batch["v"]), dev(batch["sinks"]), out)
    torch.cuda.synchronize()
    return out


def oracle_attention(batch, shape, order=None, sink_key=True, q=None, k=None, pictures=None):
    """The oracle over the chosen pictures (all by default), each on its own."""
    q = batch["q"] if q is None else q
    k = batch["k"] if k is None else k
    cu = batch["cu_seqlens"].tolist()
    pics = range(len(cu) - 1) if pictures is None else pictures
    sinks = None if batch["sinks"] is None else f64(batch["sinks"])
    refs, rows = [], []
    for s in pics:
        a, b = cu[s], cu[s + 1]
        o = None if order is None else order[a:b]
        refs.append(oracle.vit_attn(f64(q[a:b]), f64(k[a:b]), f64(batch["v"][a:b]), [0, b - a],
                                    window=shape.window, tau=shape.softmax_scale, order=o, sink_key=sink_key,
                                    sinks=sinks))
        rows.append(np.arange(a, b))
    return np.concatenate(rows), np.concatenate(refs)


# ------------------------------------------------------------------ 2D RoPE
@pytest.mark.parametrize("inplace", [False, True])
def test_vit_rope_2d_against_oracle(inplace):
    grids = [wl.VIT_PAGE_GRID, (8, 6), (2, 2)]
    note(f"vit_rope_2d grids {grids} inplace={inplace}")
    b = wl.vit_batch(seed=31, grids=grids)
    shape = wl.vit_shape()
    row, col, _ = layouts(grids, lib=True)
    q, k = dev(b["q"]), dev(b["k"])
    qo, ko = (q.clone(), k.clone()) if inplace else (torch.empty_like(q), torch.empty_like(k))
    qi, ki = (qo, ko) if inplace else (q, k)
    hsw.hsw_vit_rope_2d(shape, q.shape[0], qi, ki, torch.from_numpy(row).to(DEV), torch.from_numpy(col).to(DEV),
                        qo, ko)
    torch.cuda.synchronize()
    orow, ocol, _ = layouts(grids, lib=False)
    for x, y in ((b["q"], qo), (b["k"], ko)):
        ref = oracle.rope_2d(f64(x), orow, ocol, wl.VIT_THETA)
        err = np.abs(f64(y) - ref)
        tol = bf16_ulp(ref) + 1e-6
        assert np.all(err <= tol), f"rope_2d off by {float((err - tol).max()):.3e} beyond one bf16 ulp"


def test_vit_rope_2d_k_only_leaves_q_alone():
    note("vit_rope_2d k only")
    b = wl.vit_batch(seed=32, grids=[(4, 6)])
    shape = wl.vit_shape()
    row, col, _ = layouts([(4, 6)], lib=True)
    k = dev(b["k"])
    ko = torch.empty_like(k)
    hsw.hsw_vit_rope_2d(shape, 24, None, k, torch.from_numpy(row).to(DEV), torch.from_numpy(col).to(DEV), None, ko)
    torch.cuda.synchronize()
    ref = oracle.rope_2d(f64(b["k"]), row, col, wl.VIT_THETA)
    assert np.all(np.abs(f64(ko) - ref) <= bf16_ulp(ref) + 1e-6)


# ---------------------------------------------------------------- attention
GRIDS = [wl.VIT_PAGE_GRID, (8, 6), (2, 2), (8, 8), (2, 66), (16, 10)]   # 1008, 48, 4, 64, 132, 160 tokens


@pytest.mark.parametrize("mode", ["full", "window_row", "window_col", "window_col_nosinkkey_learned"])
def test_vit_attention_modes(mode):
    note(f"vit_attention {mode} grids {GRIDS}")
    learned = mode.endswith("learned")
    b = wl.vit_batch(seed=33, grids=GRIDS, with_sinks=learned)
    shape = wl.vit_shape(window=0 if mode == "full" else 64)
    sink_key = mode in ("window_row", "window_col")
    use_col = mode.startswith("window_col")
    order_lib = layouts(GRIDS, lib=True)[2] if use_col else None
    order_ref = layouts(GRIDS, lib=False)[2] if use_col else None
    out = run_attention(b, shape, order_lib, sink_key)
    idx, ref = oracle_attention(b, shape, order_ref, sink_key)
    ma, mr = assert_close(f64(out)[idx], ref, what=f"vit_attention {mode}")
    print(f"vit_attention {mode}: max_abs={ma:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("hq,hkv", [(16, 16), (16, 8), (16, 2), (32, 2)])
def test_vit_attention_groups(hq, hkv):
    note(f"vit_attention groups {hq}/{hkv}")
    grids = [(8, 12), (2, 2), (10, 14)]
    b = wl.vit_batch(seed=34, grids=grids, hq=hq, hkv=hkv)
    for window in (64, 0):
        shape = wl.vit_shape(hq, hkv, window=window)
        order_lib = layouts(grids, lib=True)[2]
        order_ref = layouts(grids, lib=False)[2]
        out = run_attention(b, shape, order_lib, True)
        idx, ref = oracle_attention(b, shape, order_ref, True)
        ma, mr = assert_close(f64(out)[idx], ref, what=f"vit_attention G={hq // hkv} window={window}")
        print(f"vit_attention G={hq // hkv} window={window}: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_vit_attention_peaked_and_arbitrary_order():
    """Sharp attention (q scaled by 6: the running max is raised across
    chunks) and an arbitrary permutation as the order (its first token, not
    token 0, is the sink key)."""
    note("vit_attention peaked, random order")
    grids = [(20, 24), (6, 4)]
    b = wl.vit_batch(seed=35, grids=grids, q_scale=6.0)
    g = np.random.default_rng(35)
    order = np.concatenate([g.permutation(n) for n in b["lens"]]).astype(np.int32)
    for window in (64, 0):
        shape = wl.vit_shape(window=window)
        out = run_attention(b, shape, order, True)
        idx, ref = oracle_attention(b, shape, order, True)
        ma, mr = assert_close(f64(out)[idx], ref, what=f"vit_attention peaked window={window}")
        print(f"vit_attention peaked window={window}: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_vit_attention_empty_pictures_and_batch_independence():
    """A zero-token picture between others writes nothing; each picture's
    output equals that picture run alone (bitwise)."""
    note("vit_attention empty picture, batch independence")
    grids = [(8, 10), (0, 0), (6, 6)]
    b = wl.vit_batch(seed=36, grids=grids)
    shape = wl.vit_shape()
    out = run_attention(b, shape, None, True)
    idx, ref = oracle_attention(b, shape, None, True, pictures=[0, 2])
    assert_close(f64(out)[idx], ref, what="vit_attention with an empty picture")
    alone = wl.vit_batch(seed=36, grids=grids)
    cu = b["cu_seqlens"].tolist()
    for s in (0, 2):
        a, c = cu[s], cu[s + 1]
        one = dict(q=alone["q"][a:c], k=alone["k"][a:c], v=alone["v"][a:c],
                   cu_seqlens=torch.tensor([0, c - a]), lens=[c - a], sinks=None)
        o1 = run_attention(one, shape, None, True)
        assert torch.equal(o1, out[a:c])


def test_vit_rope_then_attention_chain():
    """The attention step of a window block as the encoder runs it: 2D RoPE of
    q and k, then windowed attention in column order with the sink key; the
    attention is gated on the rotated bf16 tensors it consumed, the chain
    from the raw inputs is reported."""
    note("vit rope + attention chain")
    grids = [wl.VIT_PAGE_GRID]
    b = wl.vit_batch(seed=37, grids=grids)
    shape = wl.vit_shape()
    row, col, order = layouts(grids, lib=True)
    q, k = dev(b["q"]), dev(b["k"])
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    hsw.hsw_vit_rope_2d(shape, q.shape[0], q, k, torch.from_numpy(row).to(DEV), torch.from_numpy(col).to(DEV),
                        qr, kr)
    out = run_attention(b, shape, order, True, q=qr, k=kr)
    orow, ocol, oorder = layouts(grids, lib=False)
    idx, ref = oracle_attention(b, shape, oorder, True, q=qr.cpu(), k=kr.cpu())
    ma, mr = assert_close(f64(out)[idx], ref, what="vit chain (gated on the rotated tensors)")
    qr64 = oracle.rope_2d(f64(b["q"]), orow, ocol, wl.VIT_THETA)
    kr64 = oracle.rope_2d(f64(b["k"]), orow, ocol, wl.VIT_THETA)
    ref_raw = oracle.vit_attn(qr64, kr64, f64(b["v"]), [0, q.shape[0]], window=64, tau=shape.softmax_scale,
                              order=oorder, sink_key=True)
    ma2, mr2 = errors(f64(out), ref_raw)
    print(f"vit chain: gated max_abs={ma:.2e} mean_rel={mr:.2e}; from raw q/k max_abs={ma2:.2e} mean_rel={mr2:.2e}")


@pytest.mark.parametrize("mode", ["window_col", "full"])
def test_vit_attention_full_size_sampled(mode):
    """The bench workload (16 pictures of 64 x 64 patches, 65536 tokens,
    16 q / 4 KV heads): two pictures checked whole against the oracle."""
    note(f"vit_attention full size {mode}")
    grids = wl.VIT_BENCH_GRIDS
    b = wl.vit_batch(seed=38, grids=grids, device=DEV)
    shape = wl.vit_shape(window=0 if mode == "full" else 64)
    order_lib = layouts(grids, lib=True)[2] if mode != "full" else None
    order_ref = layouts(grids, lib=False)[2] if mode != "full" else None
    out = run_attention(b, shape, order_lib, mode != "full")
    bc = {kk: (vv.cpu() if isinstance(vv, torch.Tensor) else vv) for kk, vv in b.items()}
    pics = [0, 15] if mode != "full" else [7]
    idx, ref = oracle_attention(bc, shape, order_ref, mode != "full", pictures=pics)
    ma, mr = assert_close(f64(out[torch.from_numpy(idx).to(DEV)]), ref, what=f"vit full size {mode}")
    print(f"vit_attention full size {mode} (pictures {pics}): max_abs={ma:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("window", [64, 0])
def test_vit_attention_values_beyond_fp16_range(window):
    """V rows with abs ~ 1e5 (outside fp16) in some chunks, the sink row
    among them: those chunks take the exact bf16 path, the rest fp16; the
    result still matches the oracle."""
    note(f"vit_attention large V window={window}")
    grids = [(20, 24), (8, 18)]
    b = wl.vit_batch(seed=39, grids=grids)
    v = b["v"].float()
    v[0] *= 1.0e5 / 4           # the first picture's token 0: the sink key of its later windows
    v[300:310] *= 1.0e5 / 4     # a run of rows inside one chunk / window
    b["v"] = v.to(torch.bfloat16)
    assert float(b["v"].float().abs().max()) >= 65536
    shape = wl.vit_shape(window=window)
    order_lib = layouts(grids, lib=True)[2]
    order_ref = layouts(grids, lib=False)[2]
    out = run_attention(b, shape, order_lib, True)
    idx, ref = oracle_attention(b, shape, order_ref, True)
    scale = float(np.abs(ref).max())
    ma, mr = assert_close(f64(out)[idx], ref, max_abs=2e-2 * scale, what=f"vit large V window={window}")
    print(f"vit_attention large V window={window}: max_abs={ma:.2e} (output scale {scale:.1e}) mean_rel={mr:.2e}")


def test_vit_attention_clamps_out_of_range_order_entries():
    """Order entries outside the picture are clamped into it (the header's
    contract: wrong rows, never out-of-bounds accesses): the output of every
    token that occurs once in the clamped order matches the oracle given the
    clamped order."""
    note("vit_attention out-of-range order entries")
    grids = [(8, 12), (6, 6)]
    b = wl.vit_batch(seed=40, grids=grids)
    order = layouts(grids, lib=True)[2].copy()
    order[5] = -3                 # picture 0
    order[70] = 10_000
    order[96 + 7] = 36            # picture 1 has 36 tokens: one past the end
    cu = b["cu_seqlens"].tolist()
    clamped = order.copy()
    for s in range(len(grids)):
        clamped[cu[s]:cu[s + 1]] = np.clip(order[cu[s]:cu[s + 1]], 0, cu[s + 1] - cu[s] - 1)
    shape = wl.vit_shape()
    out = run_attention(b, shape, order, True)
    idx, ref = oracle_attention(b, shape, clamped, True)
    once = []
    for s in range(len(grids)):
        local = clamped[cu[s]:cu[s + 1]]
        counts = np.bincount(local, minlength=cu[s + 1] - cu[s])
        once += [cu[s] + t for t in range(cu[s + 1] - cu[s]) if counts[t] == 1]
    once = np.array(once)
    pos = {int(r): i for i, r in enumerate(idx)}
    sel = np.array([pos[int(r)] for r in once])
    ma, mr = assert_close(f64(out)[once], ref[sel], what="vit_attention clamped order")
    print(f"vit_attention clamped order ({len(once)} tokens checked): max_abs={ma:.2e} mean_rel={mr:.2e}")


# ------------------------------------------------ fused 2D RoPE (window blocks)
def run_window_rope(batch, shape, row, col, order=None, sink_key=True):
    T = batch["q"].shape[0]
    out = torch.full((T, shape.n_q_heads, 64), SENTINEL, dtype=torch.bfloat16, device=DEV)
    od = None if order is None else torch.from_numpy(order).to(DEV)
    hsw.hsw_vit_window_attention_rope(shape, len(batch["lens"]), max(batch["lens"]), dev(batch["cu_seqlens"]), od,
                                      int(sink_key), torch.from_numpy(row).to(DEV), torch.from_numpy(col).to(DEV),
                                      dev(batch["q"]), dev(batch["k"]), dev(batch["v"]), dev(batch["sinks"]), out)
    torch.cuda.synchronize()
    return out


def rotated(batch, shape, row, col):
    q, k = dev(batch["q"]), dev(batch["k"])
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    hsw.hsw_vit_rope_2d(shape, q.shape[0], q, k, torch.from_numpy(row).to(DEV), torch.from_numpy(col).to(DEV),
                        qr, kr)
    return qr, kr


@pytest.mark.parametrize("case", ["col_sinkkey", "row_sinkkey", "col_learned_sinks"])
@pytest.mark.parametrize("hq,hkv", [(16, 4), (16, 16), (16, 8), (16, 2), (16, 1)])
def test_vit_window_attention_rope_bitwise_equals_rope_then_attention(case, hq, hkv):
    """The fused call forms each window token's angles and rotates q and k
    with the 2D RoPE call's own arithmetic: its output is byte-identical to
    hsw_vit_rope_2d then hsw_vit_attention (window 64), for every group size,
    both orders, the sink key or learned sinks, and pictures whose last
    window is partial; and it is held to the oracle fed the rotated bf16
    tensors (the bytes both paths attend over)."""
    note(f"vit window rope fused {case} {hq}/{hkv}")
    grids = [wl.VIT_PAGE_GRID, (8, 6), (2, 2), (2, 66), (16, 10)]   # 1008, 48, 4, 132, 160 tokens
    learned = case.endswith("learned_sinks")
    b = wl.vit_batch(seed=41, grids=grids, hq=hq, hkv=hkv, with_sinks=learned)
    shape = wl.vit_shape(hq, hkv, 64)
    row, col, order = layouts(grids, lib=True)
    use_col = case.startswith("col")
    sink_key = case.endswith("sinkkey")
    qr, kr = rotated(b, shape, row, col)
    out_u = run_attention(b, shape, order if use_col else None, sink_key, q=qr, k=kr)
    out_f = run_window_rope(b, shape, row, col, order if use_col else None, sink_key)
    assert torch.equal(out_f, out_u), "fused window attention differs from RoPE + attention"
    oorder = layouts(grids, lib=False)[2] if use_col else None
    idx, ref = oracle_attention(b, shape, oorder, sink_key, q=qr.cpu(), k=kr.cpu())
    ma, mr = assert_close(f64(out_f)[idx], ref, what=f"vit window rope fused {case} {hq}/{hkv}")
    print(f"vit window rope fused {case} {hq}/{hkv}: bitwise equal; max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_vit_window_attention_rope_full_size():
    """The bench workload (16 pictures of 64 x 64 patches, column order, the
    sink key): the fused call byte-identical to the two calls, and sampled
    windows held to the oracle."""
    note("vit window rope fused, 16 x 4096 tokens")
    grids = wl.VIT_BENCH_GRIDS
    b = wl.vit_batch(seed=42, grids=grids)
    shape = wl.vit_shape()
    row, col, order = layouts(grids, lib=True)
    qr, kr = rotated(b, shape, row, col)
    out_u = run_attention(b, shape, order, True, q=qr, k=kr)
    out_f = run_window_rope(b, shape, row, col, order, True)
    assert torch.equal(out_f, out_u)
    oorder = layouts(grids, lib=False)[2]
    idx, ref = oracle_attention(b, shape, oorder, True, q=qr.cpu(), k=kr.cpu(), pictures=[0, 15])
    assert_close(f64(out_f)[idx], ref, what="vit window rope fused full size")
