"""GPU parity: every C-ABI call on cuda:0 against the fp64 oracle fed the exact
tensors that call consumed ("bf16 in"), element by element.

Bars: max_abs <= 2e-2 and mean_rel <= 2e-3 for floating outputs (mean_rel is
the L1 ratio sum|y - r| / sum|r| over a call's outputs); slot / row indices
bit-exact; K written by RoPE within one bf16 ulp of the rounded fp64 value;
pass-through dims, V and untouched cache rows bitwise unchanged; the fp32
workload (logits near -25, sinks near +1) to mean_rel <= 1e-5.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, bf16_ulp, f64, linear_kv_from_ring, note, shape_kw
from parity import assert_close, errors

pytestmark = pytest.mark.gpu

hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw")
from hybrid_sliding_window_amd import workloads as wl  # noqa: E402

RING, POOL, STAGING = hsw.HSW_DST_RING, hsw.HSW_DST_POOL, hsw.HSW_DST_STAGING
SENTINEL = -7.25  # exactly representable in bf16 and fp32


def dev(t):
    return None if t is None else t.to(DEV)


def check_rope_values(x_in, y_gpu, pos, theta, rope_dim=64, what=""):
    """y_gpu against the fp64 rotation of exactly the input x_in: rotated dims
    within one bf16 ulp (+ fp32 slack), pass-through dims bitwise."""
    x = f64(x_in)
    ref = oracle.rope(x, pos, theta, rope_dim)
    y = f64(y_gpu)
    assert np.array_equal(y[..., rope_dim:], x[..., rope_dim:]), f"{what}: pass-through dims changed"
    half = rope_dim // 2
    mag = np.abs(x[..., :half]) + np.abs(x[..., half:rope_dim])
    mag = np.concatenate([mag, mag], axis=-1)
    d = np.abs(y[..., :rope_dim] - ref[..., :rope_dim])
    tol = bf16_ulp(ref[..., :rope_dim]) + 1e-6 * mag
    bad = d > tol
    assert not bad.any(), f"{what}: {bad.sum()} rotated values off by more than 1 bf16 ulp (max {d.max():.3e})"
    return float((d == 0).mean())


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("model", ["flash", "pro"])
@pytest.mark.parametrize("kind", [RING, POOL, STAGING])
def test_rope_kv_write(kind, model):
    note(f"rope kind={kind} {model}")
    m = wl.MODELS[model]
    shape = (wl.full_shape(m.n_q_heads, m.full_kv_heads, value_scale=m.value_scale) if kind == POOL
             else wl.swa_shape(m.n_q_heads, m.swa_kv_heads, value_scale=m.value_scale))
    hq, hkv = shape.n_q_heads, shape.n_kv_heads
    g = wl.gen(21 + kind)
    special = [0, 1, 127, 128, 196608, 200000, 205000, 262143, 524287, 524288]
    if kind == RING:
        T = 300
        pos = torch.cat([torch.tensor(special), torch.randint(0, 524289, (T - len(special),), generator=g)])
        seq = torch.arange(T, dtype=torch.int32)
        seq[-1] = T + 5                      # outside the ring: must be skipped, index -1
        cap = T
        seq_base = None
        kdst = torch.full((cap, hkv, 128, 192), SENTINEL, dtype=torch.bfloat16)
        vdst = torch.full((cap, hkv, 128, 128), SENTINEL, dtype=torch.bfloat16)
    elif kind == POOL:
        starts = [0, 130000, 199960, 524288 - 74]
        T = 75 * len(starts)
        pos = torch.cat([torch.arange(b, b + 75) for b in starts])
        seq = torch.repeat_interleave(torch.arange(len(starts), dtype=torch.int32), 75)
        seq_base = torch.tensor([75 * i - b for i, b in enumerate(starts)], dtype=torch.int64)
        cap = T + 10
        kdst = torch.full((cap, hkv, 192), SENTINEL, dtype=torch.bfloat16)
        vdst = torch.full((cap, hkv, 128), SENTINEL, dtype=torch.bfloat16)
    else:
        T = 333
        pos = torch.randint(0, 524289, (T,), generator=g)
        pos[:len(special)] = torch.tensor(special)
        seq = None
        seq_base = None
        cap = T + 7
        kdst = torch.full((cap, hkv, 192), SENTINEL, dtype=torch.bfloat16)
        vdst = torch.full((cap, hkv, 128), SENTINEL, dtype=torch.bfloat16)
    pos = pos.to(torch.int64)
    q = wl.randn((T, hq, 192), g)
    k = wl.randn((T, hkv, 192), g)
    v = wl.randn((T, hkv, 128), g)
    d_q, d_k, d_v, d_pos = dev(q), dev(k), dev(v), dev(pos)
    d_seq, d_base = dev(seq), dev(seq_base)
    d_kdst, d_vdst = dev(kdst), dev(vdst)
    q_rot = torch.empty_like(d_q)
    idx = torch.full((T,), -99, dtype=torch.int64, device=DEV)
    hsw.hsw_rope_partial_kv_write(shape, T, d_q, d_k, d_v, d_pos, d_seq, kind, d_kdst, d_vdst, cap,
                                  d_base, q_rot, idx)
    torch.cuda.synchronize()
    P = pos.numpy()
    # indices: exact
    want = []
    for t in range(T):
        if kind == RING:
            s = int(seq[t])
            want.append(oracle.dst_index(oracle.RING, t, int(P[t])) if s < cap else -1)
        elif kind == POOL:
            want.append(oracle.dst_index(oracle.POOL, t, int(P[t]), int(seq_base[int(seq[t])])))
        else:
            want.append(oracle.dst_index(oracle.STAGING, t, int(P[t])))
    got = idx.cpu().numpy()
    assert np.array_equal(got, np.array(want)), "destination indices differ"
    frac_q = check_rope_values(q, q_rot, P, shape.rope_theta, what="q_rot")
    kd, vd = kdst.clone(), vdst.clone()
    gk, gv = d_kdst.cpu(), d_vdst.cpu()
    written = np.zeros(gk.shape[:-1], bool)
    for t in range(T):
        if want[t] < 0:
            continue
        if kind == RING:
            s = int(seq[t])
            sel_k, sel_v = gk[s, :, want[t]], gv[s, :, want[t]]
            written[s, :, want[t]] = True
        else:
            sel_k, sel_v = gk[want[t]], gv[want[t]]
            written[want[t]] = True
        check_rope_values(k[t:t + 1], sel_k[None], P[t:t + 1], shape.rope_theta, what=f"k[{t}]")
        assert torch.equal(sel_v, v[t]), f"v[{t}] not copied bit-exactly"
    # everything not written keeps the sentinel bytes
    assert torch.equal(gk[torch.from_numpy(~written)], kd[torch.from_numpy(~written)])
    assert torch.equal(gv[torch.from_numpy(~written)], vd[torch.from_numpy(~written)])
    print(f"rope kind={kind} {model}: q_rot bitwise-equal fraction {frac_q:.3f}")


def test_rope_fp32_logit_shift_layer():
    """fp32 storage (the logit-shift workload): rotation within fp32 rounding."""
    note("rope fp32")
    d = wl.logit_shift_layer()
    shape = d["shape"]
    T = d["q"].shape[0]
    q_rot = torch.empty_like(dev(d["q"]))
    kst = torch.empty_like(dev(d["k"]))
    vst = torch.empty_like(dev(d["v"]))
    hsw.hsw_rope_partial_kv_write(shape, T, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["pos"]), None,
                                  STAGING, kst, vst, T, None, q_rot)
    torch.cuda.synchronize()
    P = d["pos"].numpy()
    for x, y in ((d["q"], q_rot), (d["k"], kst)):
        ref = oracle.rope(f64(x), P, shape.rope_theta)
        assert np.abs(f64(y) - ref).max() <= 2e-6 * np.abs(ref).max()
    assert torch.equal(vst.cpu(), d["v"])


# ------------------------------------------------------------ SWA decode
def run_swa_decode(batch):
    shape = batch["shape"]
    S = batch["pos"].shape[0]
    kring, vring = dev(batch["kring"]), dev(batch["vring"])
    q_rot = torch.empty_like(dev(batch["q"]))
    idx = torch.empty(S, dtype=torch.int64, device=DEV)
    hsw.hsw_rope_partial_kv_write(shape, S, dev(batch["q"]), dev(batch["k"]), dev(batch["v"]),
                                  dev(batch["pos"]), dev(batch["seq"]), RING, kring, vring, S, None,
                                  q_rot, idx)
    out = torch.empty((S, shape.n_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    sinks = dev(batch["sinks"])
    hsw.hsw_swa_decode(shape, S, dev(batch["pos"]), q_rot, kring, vring, sinks, out)
    torch.cuda.synchronize()
    return q_rot, kring, vring, out, idx


@pytest.mark.parametrize("model", ["flash", "pro"])
@pytest.mark.parametrize("case", ["small_positions", "decode_256_seqs"])
def test_swa_decode(case, model):
    mk = wl.model_kw(wl.MODELS[model], "swa")
    if case == "small_positions":
        positions = [0, 1, 2, 5, 63, 126, 127, 128, 129, 255, 1000, 524288]
        batch = wl.swa_decode_batch(seed=31, n_seqs=len(positions), positions=positions, **mk)
    else:
        batch = wl.swa_decode_batch(seed=3, **mk)   # 256 sequences at positions U{128..524288}
    note(f"swa_decode {case} {model}")
    shape = batch["shape"]
    ring_before = batch["kring"].clone()
    q_rot, kring, vring, out, idx = run_swa_decode(batch)
    P = batch["pos"].numpy()
    assert np.array_equal(idx.cpu().numpy(), P % 128)
    # only slot P mod 128 of each sequence changed
    kr = kring.cpu()
    for s in range(len(P)):
        other = torch.ones(128, dtype=torch.bool)
        other[int(P[s]) % 128] = False
        assert torch.equal(kr[s][:, other], ring_before[s][:, other])
    ref = oracle.ring_decode(f64(q_rot), P, f64(kring), f64(vring), sinks=f64(batch["sinks"]), **shape_kw(shape))
    ma, mr = assert_close(f64(out), ref, what=f"swa_decode {case}")
    # chain from the raw inputs (reported, not gated)
    qr = oracle.rope(f64(batch["q"]), P, shape.rope_theta)
    kn = oracle.rope(f64(batch["k"]), P, shape.rope_theta)
    kring64, vring64 = f64(batch["kring"]), f64(batch["vring"])
    for s in range(len(P)):
        kring64[s, :, P[s] % 128] = kn[s]
        vring64[s, :, P[s] % 128] = f64(batch["v"])[s]
    chain = oracle.ring_decode(qr, P, kring64, vring64, sinks=f64(batch["sinks"]), **shape_kw(shape))
    cma, cmr = errors(f64(out), chain)
    print(f"swa_decode {case} {model}: bf16-in max_abs={ma:.2e} mean_rel={mr:.2e}; chain max_abs={cma:.2e} mean_rel={cmr:.2e}")


def test_swa_decode_batch_order_bitwise():
    """A row depends only on its own inputs: permuting the batch permutes the
    output bytes (colibri 'System One mode': rows must not depend on others)."""
    note("swa_decode batch order")
    batch = wl.swa_decode_batch(seed=33, n_seqs=40)
    _, _, _, out, _ = run_swa_decode(batch)
    perm = torch.randperm(40, generator=wl.gen(34))
    pb = {k: (v[perm] if isinstance(v, torch.Tensor) and v.shape[:1] == (40,) else v) for k, v in batch.items()}
    pb["seq"] = torch.arange(40, dtype=torch.int32)
    _, _, _, out_p, _ = run_swa_decode(pb)
    assert torch.equal(out_p.cpu(), out.cpu()[perm])


# ----------------------------------------------------------- SWA prefill
def run_swa_prefill(batch):
    shape = batch["shape"]
    T = batch["q"].shape[0]
    S = batch["start_pos"].shape[0]
    lens = (batch["cu_seqlens"][1:] - batch["cu_seqlens"][:-1])
    q_rot = torch.empty_like(dev(batch["q"]))
    kst = torch.empty_like(dev(batch["k"]))
    vst = torch.empty_like(dev(batch["v"]))
    hsw.hsw_rope_partial_kv_write(shape, T, dev(batch["q"]), dev(batch["k"]), dev(batch["v"]),
                                  dev(batch["pos"]), None, STAGING, kst, vst, T, None, q_rot)
    kring, vring = dev(batch["kring"]), dev(batch["vring"])
    kring_before, vring_before = kring.cpu(), vring.cpu()
    out = torch.full((T, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    hsw.hsw_swa_prefill(shape, S, int(lens.max()) + 3, dev(batch["cu_seqlens"]), dev(batch["start_pos"]),
                        q_rot, kst, vst, kring, vring, dev(batch["sinks"]), out)
    torch.cuda.synchronize()
    return q_rot, kst, vst, kring_before, vring_before, kring, vring, out


def check_ring_commit(batch, kst, vst, kring_before, vring_before, kring, vring):
    cu = batch["cu_seqlens"].tolist()
    st = batch["start_pos"].tolist()
    kr, vr, ks, vs = kring.cpu(), vring.cpu(), kst.cpu(), vst.cpu()
    for s in range(len(st)):
        n = cu[s + 1] - cu[s]
        written = torch.zeros(128, dtype=torch.bool)
        for t in range(max(0, n - 128), n):
            slot = (st[s] + t) % 128
            written[slot] = True
            assert torch.equal(kr[s, :, slot], ks[cu[s] + t]) and torch.equal(vr[s, :, slot], vs[cu[s] + t])
        assert torch.equal(kr[s][:, ~written], kring_before[s][:, ~written])
        assert torch.equal(vr[s][:, ~written], vring_before[s][:, ~written])


def oracle_swa_prefill_rows(batch, q_rot, kst, vst, kring_before, vring_before, rows=None):
    """Oracle outputs for chunk rows (all, or a per-sequence sample)."""
    shape = batch["shape"]
    cu = batch["cu_seqlens"].tolist()
    st = batch["start_pos"].tolist()
    kr0, vr0 = f64(kring_before), f64(vring_before)
    sinks = f64(batch["sinks"])
    outs = []
    for s in range(len(st)):
        sel = np.arange(cu[s], cu[s + 1]) if rows is None else np.asarray(rows[s])
        if sel.size == 0:
            continue
        ks, vs = f64(kst[cu[s]:cu[s + 1]]), f64(vst[cu[s]:cu[s + 1]])
        k, v, kpos0 = linear_kv_from_ring(kr0[s], vr0[s], st[s], ks, vs)
        qpos = st[s] + (sel - cu[s])
        qsel = f64(q_rot[torch.from_numpy(sel).to(q_rot.device)])
        outs.append((sel, oracle.attn_linear(qsel, qpos, k, v, kpos0, window=128, sinks=sinks,
                                             **shape_kw(shape))))
    return outs


def test_swa_prefill_values_beyond_fp16_range():
    """V beyond the fp16 range in whole rows (chunk rows and ring rows) and
    in single columns: the column blocks holding them keep bf16, the rest of
    each 32-key chunk goes through fp16, and the result matches."""
    note("swa_prefill large V")
    batch = wl.swa_prefill_batch(seed=45, n_seqs=2, seqlens=(400, 150), start_pos=(300, 0))
    v = batch["v"].float()
    v[7::41] *= 2.0e5                      # whole rows of the chunk
    v[20::23, :, 70] *= -1.5e5             # one column: column block 2 only
    batch["v"] = v.to(torch.bfloat16)
    vr = batch["vring"].float()
    vr[0, :, 5::37] *= 3.0e5               # ring rows read by the first sequence's early rows
    batch["vring"] = vr.to(torch.bfloat16)
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    check_ring_commit(batch, kst, vst, kb, vb, kring, vring)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(batch, q_rot, kst, vst, kb, vb)])
    ma, mr = assert_close(f64(out), ref, max_abs=2e-2 * float(np.abs(ref).max()), what="swa_prefill large V")
    print(f"swa_prefill large V: max_abs={ma:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("hq,hkv,lam", [(64, 8, wl.VALUE_SCALE_FLASH), (128, 8, wl.VALUE_SCALE_PRO),
                                        (32, 8, wl.VALUE_SCALE_FLASH)])
def test_swa_prefill_ragged(hq, hkv, lam):
    note(f"swa_prefill ragged hq={hq} hkv={hkv}")
    batch = wl.swa_prefill_batch(seed=41, n_seqs=3, seqlens=(300, 17, 1000), start_pos=(0, 5000, 130),
                                 hq=hq, hkv=hkv, value_scale=lam)
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    check_ring_commit(batch, kst, vst, kb, vb, kring, vring)
    got = f64(out)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(batch, q_rot, kst, vst, kb, vb)])
    ma, mr = assert_close(got, ref, what="swa_prefill ragged")
    print(f"swa_prefill ragged hq={hq}: max_abs={ma:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_swa_prefill_full_size(model):
    """4 x 8192 from position 0: every row and head of every sequence against
    the oracle, plus the ring commit."""
    note(f"swa_prefill 4x8192 all rows {model}")
    batch = wl.swa_prefill_batch(seed=2, **wl.model_kw(wl.MODELS[model], "swa"))
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    check_ring_commit(batch, kst, vst, kb, vb, kring, vring)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(batch, q_rot, kst, vst, kb, vb)])
    ma, mr = assert_close(f64(out), ref, what=f"swa_prefill 4x8192 {model}")
    print(f"swa_prefill 4x8192 all {out.shape[0]} rows {model}: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_logit_shift_layer_fp32_chain():
    """One windowed layer in fp32 (1 x 512, 4/1 heads, logits ~ -25, sinks ~ +1):
    rope + windowed prefill against the oracle from the raw inputs."""
    note("fp32 logit-shift layer")
    d = wl.logit_shift_layer()
    shape = d["shape"]
    T = 512
    q_rot = torch.empty_like(dev(d["q"]))
    kst = torch.empty_like(dev(d["k"]))
    vst = torch.empty_like(dev(d["v"]))
    hsw.hsw_rope_partial_kv_write(shape, T, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["pos"]), None,
                                  STAGING, kst, vst, T, None, q_rot)
    kring = torch.zeros((1, 1, 128, 192), dtype=torch.float32, device=DEV)
    vring = torch.zeros((1, 1, 128, 128), dtype=torch.float32, device=DEV)
    out = torch.empty((T, 4, 128), dtype=torch.float32, device=DEV)
    hsw.hsw_swa_prefill(shape, 1, T, dev(d["cu_seqlens"]), dev(d["start_pos"]), q_rot, kst, vst,
                        kring, vring, dev(d["sinks"]), out)
    torch.cuda.synchronize()
    P = d["pos"].numpy()
    qr = oracle.rope(f64(d["q"]), P, shape.rope_theta)
    kr = oracle.rope(f64(d["k"]), P, shape.rope_theta)
    ref = oracle.attn_linear(qr, P, kr, f64(d["v"]), 0, window=128, sinks=f64(d["sinks"]), **shape_kw(shape))
    ma, mr = assert_close(f64(out), ref, mean_rel=1e-5, what="fp32 chain")
    print(f"fp32 logit-shift chain: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_windowed_calls_at_positions_beyond_2_31():
    """Windowed positions are int64 (the ring needs only p mod 128): a chunk
    that crosses 2^31, one past 2^33, their fused q-RoPE form and decodes at
    such positions, all against the oracle (the fused chain from the raw q
    rotated in fp64)."""
    note("windowed calls past 2^31")
    starts = (2 ** 31 - 50, 2 ** 33 + 3, 2 ** 31 + 1)
    batch = wl.swa_prefill_batch(seed=48, n_seqs=3, seqlens=(300, 140, 1), start_pos=starts)
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    check_ring_commit(batch, kst, vst, kb, vb, kring, vring)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(batch, q_rot, kst, vst, kb, vb)])
    ma, mr = assert_close(f64(out), ref, what="swa_prefill past 2^31")
    check_rope_values(batch["q"], q_rot, batch["pos"].numpy(), wl.THETA_SWA, what="q_rot past 2^31")
    kst2, vst2, kring2, vring2, out2 = run_swa_prefill_qrope(batch)
    assert torch.equal(out2, out) and torch.equal(kring2, kring)
    positions = [2 ** 31 - 1, 2 ** 31, 2 ** 31 + 127, 2 ** 32 + 5, 2 ** 40 + 3, 2 ** 52 + 9]
    dec = wl.swa_decode_batch(seed=49, n_seqs=len(positions), positions=positions)
    q_rot_d, kring_d, vring_d, out_d, idx = run_swa_decode(dec)
    P = dec["pos"].numpy()
    assert np.array_equal(idx.cpu().numpy(), P % 128)
    ref_d = oracle.ring_decode(f64(q_rot_d), P, f64(kring_d), f64(vring_d), sinks=f64(dec["sinks"]),
                               **shape_kw(dec["shape"]))
    dma, dmr = assert_close(f64(out_d), ref_d, what="swa_decode past 2^31")
    print(f"past 2^31: prefill max_abs={ma:.2e} mean_rel={mr:.2e}; decode max_abs={dma:.2e} mean_rel={dmr:.2e}")


def test_decode_matches_prefill_row():
    """Decode at position P equals prefill row P (colibri 'Correctness':
    prefill in blocks and one token at a time agree)."""
    note("decode vs prefill row")
    batch = wl.swa_prefill_batch(seed=51, n_seqs=1, seqlens=(300,), start_pos=(0,))
    shape = batch["shape"]
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    # ring now holds positions 172..299; decode position 299 with its q_rot row
    o = torch.empty((1, 64, 128), dtype=torch.bfloat16, device=DEV)
    hsw.hsw_swa_decode(shape, 1, torch.tensor([299], device=DEV), q_rot[299:300].contiguous(), kring,
                       vring, dev(batch["sinks"]), o)
    torch.cuda.synchronize()
    assert_close(f64(o)[0], f64(out)[299], what="decode vs prefill row")


def permute_prefill_batch(batch, perm, per_seq_keys):
    """The same sequences in the order `perm`: chunk rows moved with their
    sequence, cu_seqlens and positions rebuilt, and the per-sequence tensors
    named in per_seq_keys (rings, starts, pool bases) permuted."""
    cu = batch["cu_seqlens"].tolist()
    rows = torch.cat([torch.arange(cu[s], cu[s + 1]) for s in perm]) if cu[-1] else torch.zeros(0, dtype=torch.long)
    lens = torch.tensor([cu[s + 1] - cu[s] for s in perm], dtype=torch.int64)
    pb = dict(batch)
    for k in ("q", "k", "v", "pos"):
        pb[k] = batch[k][rows]
    for k in per_seq_keys:
        pb[k] = batch[k][list(perm)]
    pb["cu_seqlens"] = torch.zeros(len(perm) + 1, dtype=torch.int64)
    pb["cu_seqlens"][1:] = torch.cumsum(lens, 0)
    pb["seq"] = torch.repeat_interleave(torch.arange(len(perm), dtype=torch.int32), lens)
    return pb, rows


def test_swa_prefill_batch_order_bitwise():
    """A prefill row depends only on its own sequence (colibri 'Correctness';
    P14): the same sequences in another order give byte-identical output
    rows and ring commits."""
    note("swa_prefill batch order")
    batch = wl.swa_prefill_batch(seed=46, n_seqs=5, seqlens=(300, 17, 0, 700, 129),
                                 start_pos=(0, 5000, 64, 130, 524000))
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    perm = [3, 0, 4, 2, 1]
    pb, rows = permute_prefill_batch(batch, perm, ("kring", "vring", "start_pos"))
    _, _, _, _, _, kring_p, vring_p, out_p = run_swa_prefill(pb)
    assert torch.equal(out_p.cpu(), out.cpu()[rows]), "output rows depend on batch order"
    assert torch.equal(kring_p.cpu(), kring.cpu()[perm]) and torch.equal(vring_p.cpu(), vring.cpu()[perm])


def test_full_prefill_batch_order_bitwise():
    """The chunked full prefill under a permutation of its sequences (pool rows
    stay where they are; the sequences' bases move with them): byte-identical
    output rows (colibri 'Correctness'; P14)."""
    note("full_prefill batch order")
    batch = wl.full_prefill_batch(seed=75, n_seqs=4, seqlens=(300, 77, 129, 1), start_pos=(3000, 100, 0, 40000))
    _, _, _, out = run_full_prefill(batch)
    perm = [2, 3, 0, 1]
    pb, rows = permute_prefill_batch(batch, perm, ("start_pos", "seq_base", "ctx_len"))
    _, _, _, out_p = run_full_prefill(pb)
    assert torch.equal(out_p.cpu(), out.cpu()[rows]), "output rows depend on batch order"


# ------------------------------------------------------- full decode
def run_full_decode(batch, chunk=2048, sinks=None):
    shape = batch["shape"]
    S = batch["ctx_len"].shape[0]
    kpool, vpool = dev(batch["kpool"]), dev(batch["vpool"])
    q_rot = torch.empty_like(dev(batch["q"]))
    rows = kpool.shape[0]
    hsw.hsw_rope_partial_kv_write(shape, S, dev(batch["q"]), dev(batch["k"]), dev(batch["v"]),
                                  dev(batch["pos"]), dev(batch["seq"]), POOL, kpool, vpool, rows,
                                  dev(batch["seq_base"]), q_rot)
    max_ctx = int(batch["ctx_len"].max())
    wsb = hsw.hsw_full_decode_workspace_bytes(shape, S, max_ctx, chunk)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=DEV)
    out = torch.empty((S, shape.n_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    hsw.hsw_full_decode_splitk(shape, S, max_ctx, dev(batch["ctx_len"]), dev(batch["seq_base"]), q_rot,
                               kpool, vpool, rows, dev(sinks), chunk, ws, wsb, out)
    torch.cuda.synchronize()
    return q_rot, kpool, vpool, out


def oracle_full_decode(batch, q_rot, kpool, vpool, seqs, sinks=None):
    shape = batch["shape"]
    L = batch["ctx_len"].tolist()
    base = batch["seq_base"].tolist()
    qr = f64(q_rot)
    res = []
    for s in seqs:
        k = f64(kpool[base[s]:base[s] + L[s]])
        v = f64(vpool[base[s]:base[s] + L[s]])
        res.append(oracle.attn_linear(qr[s:s + 1], [L[s] - 1], k, v, 0, window=0,
                                      sinks=None if sinks is None else f64(sinks), **shape_kw(shape))[0])
    return np.stack(res)


@pytest.mark.parametrize("model", ["flash", "pro"])
@pytest.mark.parametrize("chunk,with_sink", [(2048, False), (1024, False), (2048, True), (128, True)])
def test_full_decode_small(chunk, with_sink, model):
    note(f"full_decode small chunk={chunk} sink={with_sink} {model}")
    lengths = [1, 2, 127, 2047, 2048, 2049, 9000, 4097]
    batch = wl.full_decode_batch(seed=61, n_seqs=len(lengths), lengths=lengths, with_sinks=with_sink,
                                 **wl.model_kw(wl.MODELS[model], "full"))
    q_rot, kpool, vpool, out = run_full_decode(batch, chunk, batch["sinks"])
    ref = oracle_full_decode(batch, q_rot, kpool, vpool, range(len(lengths)), batch["sinks"])
    ma, mr = assert_close(f64(out), ref, what="full_decode small")
    print(f"full_decode chunk={chunk} sink={with_sink} {model}: max_abs={ma:.2e} mean_rel={mr:.2e}")


def c4_sequences(L, n=None, seed=4):
    """Sequences of the 64-sequence full decode held to the oracle: all of
    them (n None), or the shortest, the longest and n - 2 others drawn from a
    seeded generator."""
    if n is None:
        return list(range(len(L)))
    lo, hi = int(L.argmin()), int(L.argmax())
    rest = [s for s in range(len(L)) if s not in (lo, hi)]
    pick = np.random.default_rng(seed).choice(rest, n - 2, replace=False)
    return sorted({lo, hi, *map(int, pick)})


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_full_decode_full_size(model):
    """64 sequences with contexts U{32768..131072}: every head of all 64
    sequences (Flash) or of 16 including the shortest and the longest (Pro,
    whose pool is twice as large) against the oracle."""
    note(f"full_decode 64 seqs {model}")
    batch = wl.full_decode_batch(seed=4, device=DEV, **wl.model_kw(wl.MODELS[model], "full"))
    q_rot, kpool, vpool, out = run_full_decode(batch)
    seqs = c4_sequences(batch["ctx_len"].numpy(), None if model == "flash" else 16)
    ref = oracle_full_decode(batch, q_rot, kpool, vpool, seqs)
    ma, mr = assert_close(f64(out[seqs]), ref, what="full_decode 64 seqs")
    print(f"full_decode 64 seqs {model} ({len(seqs)} checked): max_abs={ma:.2e} mean_rel={mr:.2e}")


# ------------------------------------------------------ full prefill
def run_full_prefill(batch):
    shape = batch["shape"]
    T = batch["q"].shape[0]
    S = batch["start_pos"].shape[0]
    kpool, vpool = dev(batch["kpool"]), dev(batch["vpool"])
    rows = kpool.shape[0]
    q_rot = torch.empty_like(dev(batch["q"]))
    hsw.hsw_rope_partial_kv_write(shape, T, dev(batch["q"]), dev(batch["k"]), dev(batch["v"]),
                                  dev(batch["pos"]), dev(batch["seq"]), POOL, kpool, vpool, rows,
                                  dev(batch["seq_base"]), q_rot)
    lens = batch["cu_seqlens"][1:] - batch["cu_seqlens"][:-1]
    out = torch.empty((T, shape.n_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    hsw.hsw_full_prefill_chunk(shape, S, int(lens.max()), dev(batch["cu_seqlens"]), dev(batch["start_pos"]),
                               dev(batch["seq_base"]), q_rot, kpool, vpool, rows, None, out)
    torch.cuda.synchronize()
    return q_rot, kpool, vpool, out


def oracle_full_prefill(batch, q_rot, kpool, vpool, rows_per_seq):
    shape = batch["shape"]
    cu = batch["cu_seqlens"].tolist()
    st = batch["start_pos"].tolist()
    base = batch["seq_base"].tolist()
    qr = f64(q_rot)
    got_idx, refs = [], []
    for s, sel in enumerate(rows_per_seq):
        sel = np.asarray(sel)
        if sel.size == 0:
            continue
        n = st[s] + cu[s + 1] - cu[s]
        k = f64(kpool[base[s]:base[s] + n])
        v = f64(vpool[base[s]:base[s] + n])
        refs.append(oracle.attn_linear(qr[sel], st[s] + sel - cu[s], k, v, 0, window=0, **shape_kw(shape)))
        got_idx.append(sel)
    return np.concatenate(got_idx), np.concatenate(refs)


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_full_prefill_ragged(model):
    note(f"full_prefill ragged {model}")
    batch = wl.full_prefill_batch(seed=71, n_seqs=3, seqlens=(300, 77, 129), start_pos=(3000, 100, 0),
                                  **wl.model_kw(wl.MODELS[model], "full"))
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    cu = batch["cu_seqlens"].tolist()
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, [np.arange(cu[s], cu[s + 1]) for s in range(3)])
    ma, mr = assert_close(f64(out)[idx], ref, what="full_prefill ragged")
    print(f"full_prefill ragged {model}: max_abs={ma:.2e} mean_rel={mr:.2e}")


def sampled_chunk_rows(T, seed, n_random=124):
    """The first 130 rows of a chunk, its last 2 and n_random others drawn
    from a seeded generator (sorted, distinct)."""
    g = np.random.default_rng(seed)
    r = list(range(130)) + [T - 2, T - 1]
    r += list(g.choice(np.arange(130, T - 2), n_random, replace=False))
    return np.array(sorted(set(r)))


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_full_prefill_chunk_8192_after_131072_sampled(model):
    """8192-token chunk after 131072 prior rows: every head of 256 rows (the
    first 130, the last 2 and 124 random ones, which reach well over a
    hundred of the 64-row query blocks) against the oracle."""
    note(f"full_prefill 8192 @ 131072 sampled {model}")
    batch = wl.full_prefill_batch(seed=5, device=DEV, **wl.model_kw(wl.MODELS[model], "full"))
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    rows = [sampled_chunk_rows(8192, seed=5)]
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, rows)
    ma, mr = assert_close(f64(out[torch.from_numpy(idx)]), ref, what="full_prefill 8192")
    print(f"full_prefill 8192@131072 {len(idx)} rows {model}: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_full_prefill_values_beyond_fp16_range():
    """V rows with |v| ~ 1e5 (outside fp16 range) still match the oracle: no
    step of the kernel narrows V below bf16."""
    note("full_prefill large V")
    batch = wl.full_prefill_batch(seed=72, n_seqs=2, seqlens=(200, 64), start_pos=(300, 37))
    rows = batch["vpool"].shape[0]
    big = torch.arange(0, rows, 37)
    batch["vpool"][big] = (batch["vpool"][big].float() * 2.0e5).to(torch.bfloat16)
    batch["v"][5] = (batch["v"][5].float() * 3.0e5).to(torch.bfloat16)
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    cu = batch["cu_seqlens"].tolist()
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, [np.arange(cu[s], cu[s + 1]) for s in range(2)])
    ma, mr = assert_close(f64(out)[idx], ref, max_abs=2e-2 * float(np.abs(ref).max()), what="full_prefill large V")
    print(f"full_prefill large V: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_full_prefill_values_beyond_fp16_range_in_some_columns():
    """Out-of-fp16-range V confined to a few columns of some rows: the keys
    around them keep bf16 while the rest go through fp16, and the result
    still matches."""
    note("full_prefill large V in some columns")
    batch = wl.full_prefill_batch(seed=74, n_seqs=2, seqlens=(150, 90), start_pos=(250, 60))
    rows = batch["vpool"].shape[0]
    big = torch.arange(3, rows, 29)
    vp = batch["vpool"].float()
    vp[big, :, 40] *= 1.5e5          # column block 1 only
    vp[big[::2], :, 100:103] *= -3.0e5  # and block 3 in every other such row
    batch["vpool"] = vp.to(torch.bfloat16)
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    cu = batch["cu_seqlens"].tolist()
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, [np.arange(cu[s], cu[s + 1]) for s in range(2)])
    ma, mr = assert_close(f64(out)[idx], ref, max_abs=2e-2 * float(np.abs(ref).max()),
                          what="full_prefill large V in some columns")
    print(f"full_prefill large V in some columns: max_abs={ma:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_full_prefill_values_beyond_fp16_range_late_chunk(model):
    """Out-of-fp16-range V only in keys well past the first ones: query
    blocks meet it after many ordinary 64-key chunks (some only in their
    last one, some in a chunk of new rows), others never."""
    note(f"full_prefill large V in a late chunk {model}")
    batch = wl.full_prefill_batch(seed=75, n_seqs=3, seqlens=(300, 100, 40), start_pos=(500, 0, 64),
                                  **wl.model_kw(wl.MODELS[model], "full"))
    base = batch["seq_base"].tolist()
    vp = batch["vpool"].float()
    vp[base[0] + 431] *= 2.5e5          # a prior row of sequence 0
    vp[base[2] + 63, 1] *= -4.0e5       # the last prior row of sequence 2, one KV head
    batch["vpool"] = vp.to(torch.bfloat16)
    v = batch["v"].float()
    v[250] *= 3.0e5                     # a new row of sequence 0 (position 750)
    batch["v"] = v.to(torch.bfloat16)
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    cu = batch["cu_seqlens"].tolist()
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, [np.arange(cu[s], cu[s + 1]) for s in range(3)])
    ma, mr = assert_close(f64(out)[idx], ref, max_abs=2e-2 * float(np.abs(ref).max()),
                          what="full_prefill large V late chunk")
    print(f"full_prefill large V late chunk {model}: max_abs={ma:.2e} mean_rel={mr:.2e}")


# ------------------------------------------------------- degenerate cases
def test_swa_prefill_empty_and_single_token_sequences():
    """Zero-length sequences inside a batch (no rows, ring untouched),
    single-token chunks at position 0 and deep in a sequence, and a chunk
    that starts at the last ring slot and wraps it."""
    note("swa_prefill empty / single-token sequences")
    batch = wl.swa_prefill_batch(seed=43, n_seqs=6, seqlens=(0, 1, 200, 0, 129, 1),
                                 start_pos=(0, 7, 250, 40, 127, 0))
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    check_ring_commit(batch, kst, vst, kb, vb, kring, vring)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(batch, q_rot, kst, vst, kb, vb)])
    ma, mr = assert_close(f64(out), ref, what="swa_prefill degenerate")
    print(f"swa_prefill empty/single: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_full_prefill_empty_and_single_token_sequences():
    """Zero-length chunks (one of them with no pool rows at all) and
    single-token chunks, at position 0 and after prior rows."""
    note("full_prefill empty / single-token sequences")
    batch = wl.full_prefill_batch(seed=73, n_seqs=5, seqlens=(1, 0, 65, 1, 0), start_pos=(0, 500, 31, 4000, 0))
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    cu = batch["cu_seqlens"].tolist()
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, [np.arange(cu[s], cu[s + 1]) for s in range(5)])
    ma, mr = assert_close(f64(out)[idx], ref, what="full_prefill degenerate")
    print(f"full_prefill empty/single: max_abs={ma:.2e} mean_rel={mr:.2e}")


def test_general_group_size_bf16():
    """A q/KV head group of 3 (24 q heads over 8 KV heads, 12 over 4), which
    the MFMA kernels do not take: every call goes through the wave-per-row
    kernel in bf16 and must meet the same bars."""
    note("general group size: swa_prefill hq=24 hkv=8")
    b = wl.swa_prefill_batch(seed=44, n_seqs=2, seqlens=(150, 40), start_pos=(300, 0), hq=24, hkv=8)
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(b)
    check_ring_commit(b, kst, vst, kb, vb, kring, vring)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(b, q_rot, kst, vst, kb, vb)])
    assert_close(f64(out), ref, what="swa_prefill G=3")

    note("general group size: swa_decode hq=24 hkv=8")
    b = wl.swa_decode_batch(seed=45, n_seqs=5, positions=[0, 3, 127, 128, 99999], hq=24, hkv=8)
    q_rot, kring, vring, out, _ = run_swa_decode(b)
    ref = oracle.ring_decode(f64(q_rot), b["pos"].numpy(), f64(kring), f64(vring), sinks=f64(b["sinks"]),
                             **shape_kw(b["shape"]))
    assert_close(f64(out), ref, what="swa_decode G=3")

    note("general group size: full_decode hq=12 hkv=4")
    b = wl.full_decode_batch(seed=46, n_seqs=3, lengths=[1, 300, 2500], hq=12, hkv=4, with_sinks=True)
    q_rot, kpool, vpool, out = run_full_decode(b, 1024, b["sinks"])
    ref = oracle_full_decode(b, q_rot, kpool, vpool, range(3), b["sinks"])
    assert_close(f64(out), ref, what="full_decode G=3")

    note("general group size: full_prefill hq=12 hkv=4")
    b = wl.full_prefill_batch(seed=47, n_seqs=2, seqlens=(70, 33), start_pos=(200, 0), hq=12, hkv=4)
    q_rot, kpool, vpool, out = run_full_prefill(b)
    cu = b["cu_seqlens"].tolist()
    idx, ref = oracle_full_prefill(b, q_rot, kpool, vpool, [np.arange(cu[s], cu[s + 1]) for s in range(2)])
    assert_close(f64(out)[idx], ref, what="full_prefill G=3")


def test_zero_sizes_launch_nothing():
    """Calls with zero tokens, sequences or keys return without writing: on
    real device buffers every output keeps its sentinel."""
    note("zero-size calls")
    swa, full = wl.swa_shape(), wl.full_shape()
    bf = torch.bfloat16
    q = torch.zeros((4, 64, 192), dtype=bf, device=DEV)
    k8 = torch.zeros((4, 8, 192), dtype=bf, device=DEV)
    v8 = torch.zeros((4, 8, 128), dtype=bf, device=DEV)
    k4, v4 = k8[:, :4].contiguous(), v8[:, :4].contiguous()
    ring_k = torch.full((2, 8, 128, 192), SENTINEL, dtype=bf, device=DEV)
    ring_v = torch.full((2, 8, 128, 128), SENTINEL, dtype=bf, device=DEV)
    pool_k = torch.full((8, 4, 192), SENTINEL, dtype=bf, device=DEV)
    pool_v = torch.full((8, 4, 128), SENTINEL, dtype=bf, device=DEV)
    q_rot = torch.full_like(q, SENTINEL)
    out = torch.full((4, 64, 128), SENTINEL, dtype=bf, device=DEV)
    pos = torch.zeros(4, dtype=torch.int64, device=DEV)
    seq = torch.zeros(4, dtype=torch.int32, device=DEV)
    base = torch.zeros(4, dtype=torch.int64, device=DEV)
    cu = torch.zeros(5, dtype=torch.int64, device=DEV)
    lens = torch.ones(4, dtype=torch.int64, device=DEV)
    ws = torch.full((1024,), SENTINEL, dtype=torch.float32, device=DEV)
    hsw.hsw_rope_partial_kv_write(swa, 0, q, k8, v8, pos, seq, RING, ring_k, ring_v, 2, None, q_rot)
    hsw.hsw_rope_partial_kv_write(full, 0, q, k4, v4, pos, seq, POOL, pool_k, pool_v, 8, base, q_rot)
    hsw.hsw_swa_prefill(swa, 0, 16, cu, pos, q, k8, v8, ring_k, ring_v, None, out)
    hsw.hsw_swa_prefill(swa, 4, 0, cu, pos, q, k8, v8, ring_k, ring_v, None, out)
    hsw.hsw_swa_decode(swa, 0, pos, q, ring_k, ring_v, None, out)
    hsw.hsw_full_decode_splitk(full, 0, 16, lens, base, q, pool_k, pool_v, 8, None, 2048, ws, 4096, out)
    hsw.hsw_full_decode_splitk(full, 4, 0, lens, base, q, pool_k, pool_v, 8, None, 2048, ws, 4096, out)
    hsw.hsw_full_prefill_chunk(full, 0, 16, cu, pos, base, q, pool_k, pool_v, 8, None, out)
    hsw.hsw_full_prefill_chunk(full, 4, 0, cu, pos, base, q, pool_k, pool_v, 8, None, out)
    torch.cuda.synchronize()
    for name, t in [("q_rot", q_rot), ("out", out), ("ring_k", ring_k), ("ring_v", ring_v),
                    ("pool_k", pool_k), ("pool_v", pool_v), ("ws", ws)]:
        assert bool((t == SENTINEL).all()), f"{name} was written by a zero-size call"


# ------------------------------------------------------- fused q-RoPE
def test_rope_cos_sin_fp32_against_fp64():
    """The angle code itself: an fp32 RoPE call on unit vectors (x_lo = 1,
    x_hi = 0) returns exactly the fp32 cos and sin it formed, for every
    frequency at positions up to 2^52 + 5 (windowed positions are int64);
    each within 3e-7 of the fp64 rotation (angle formed and reduced in
    double, gaudi-cookbook 'The RoPE fix for large positions')."""
    note("rope cos/sin fp32 vs fp64")
    positions = [0, 1, 2, 3, 100, 127, 128, 4095, 65536, 131071, 196608, 200000, 205000, 262143,
                 524287, 524288, 1_000_003, 2 ** 24 + 5, 2 ** 31 + 7, 2 ** 33 + 3, 2 ** 40 + 9, 2 ** 52 + 5]
    T = len(positions)
    for theta in (wl.THETA_SWA, wl.THETA_FULL):
        shape = wl.Shape(1, 1, 0, theta, dtype=torch.float32)
        q = torch.zeros((T, 1, 192), dtype=torch.float32)
        q[:, :, :32] = 1.0
        k = torch.zeros((T, 1, 192), dtype=torch.float32)
        v = torch.zeros((T, 1, 128), dtype=torch.float32)
        pos = torch.tensor(positions, dtype=torch.int64)
        q_rot = torch.empty((T, 1, 192), dtype=torch.float32, device=DEV)
        kd = torch.empty((T, 1, 192), dtype=torch.float32, device=DEV)
        vd = torch.empty((T, 1, 128), dtype=torch.float32, device=DEV)
        hsw.hsw_rope_partial_kv_write(shape, T, dev(q), dev(k), dev(v), dev(pos), None, STAGING, kd, vd, T,
                                      None, q_rot)
        torch.cuda.synchronize()
        ref = oracle.rope(f64(q), pos.numpy(), theta)
        got = f64(q_rot)
        err = np.abs(got[..., :64] - ref[..., :64])
        assert err.max() <= 3e-7, f"theta={theta}: cos/sin off by {err.max():.2e} (worst position " \
                                  f"{positions[int(np.unravel_index(err.argmax(), err.shape)[0])]})"
        print(f"rope cos/sin theta={theta:.0e}: max |err| {err.max():.2e}, mean {err.mean():.2e}")


def run_swa_prefill_qrope(batch, v_in_place=False):
    """K/V-only RoPE into staging, then the prefill that rotates q itself.
    v_in_place: the RoPE call writes K only and the prefill takes v itself as
    its V staging."""
    shape = batch["shape"]
    T = batch["q"].shape[0]
    S = batch["start_pos"].shape[0]
    lens = (batch["cu_seqlens"][1:] - batch["cu_seqlens"][:-1])
    kst = torch.empty_like(dev(batch["k"]))
    v = dev(batch["v"])
    vst = v if v_in_place else torch.empty_like(v)
    hsw.hsw_rope_partial_kv_write(shape, T, None, dev(batch["k"]), None if v_in_place else v, dev(batch["pos"]),
                                  None, STAGING, kst, None if v_in_place else vst, T, None, None)
    kring, vring = dev(batch["kring"]), dev(batch["vring"])
    out = torch.full((T, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    hsw.hsw_swa_prefill_qrope(shape, S, int(lens.max()) + 3, dev(batch["cu_seqlens"]), dev(batch["start_pos"]),
                              dev(batch["q"]), kst, vst, kring, vring, dev(batch["sinks"]), out)
    torch.cuda.synchronize()
    return kst, vst, kring, vring, out


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_swa_prefill_qrope_bitwise_equals_rope_then_prefill(model):
    """The fused call rotates q with the RoPE call's own arithmetic, so its
    output, staging rows and ring commit are byte-identical to RoPE then
    hsw_swa_prefill; every output row is held to the oracle fed the bytes the
    unfused call consumed, and the error of the chain from the raw inputs
    (rotation in fp64, colibri 'What the engine implements') is reported."""
    note(f"swa_prefill_qrope bitwise {model}")
    batch = wl.swa_prefill_batch(seed=81, n_seqs=4, seqlens=(300, 17, 1000, 129),
                                 start_pos=(0, 5000, 130, 524000), **wl.model_kw(wl.MODELS[model], "swa"))
    q_rot, kst, vst, kb, vb, kring, vring, out = run_swa_prefill(batch)
    kst2, vst2, kring2, vring2, out2 = run_swa_prefill_qrope(batch)
    assert torch.equal(kst2.cpu(), kst.cpu()) and torch.equal(vst2.cpu(), vst.cpu())
    assert torch.equal(kring2.cpu(), kring.cpu()) and torch.equal(vring2.cpu(), vring.cpu())
    assert torch.equal(out2.cpu(), out.cpu()), "fused prefill differs from RoPE + prefill"
    # gate: the fused output against the oracle fed the q_rot, staging and
    # ring bytes of the unfused call (exactly what the fused call computes
    # from, by the bitwise equality above)
    ref = np.concatenate([o for _, o in oracle_swa_prefill_rows(batch, q_rot, kst, vst, kb, vb)])
    gma, gmr = assert_close(f64(out2), ref, what=f"swa_prefill_qrope {model}")
    # chain from the raw inputs: q and k rotated in fp64
    shape = batch["shape"]
    P = batch["pos"].numpy()
    qr = oracle.rope(f64(batch["q"]), P, shape.rope_theta)
    kr = oracle.rope(f64(batch["k"]), P, shape.rope_theta)
    cu, st = batch["cu_seqlens"].tolist(), batch["start_pos"].tolist()
    refs = []
    for s in range(len(st)):
        k, v, kpos0 = linear_kv_from_ring(f64(kb[s]), f64(vb[s]), st[s], kr[cu[s]:cu[s + 1]],
                                          f64(batch["v"][cu[s]:cu[s + 1]]))
        refs.append(oracle.attn_linear(qr[cu[s]:cu[s + 1]], P[cu[s]:cu[s + 1]], k, v, kpos0, window=128,
                                       sinks=f64(batch["sinks"]), **shape_kw(shape)))
    # reported, not gated: it adds the bf16 storage of the rotated q and k,
    # which the bitwise match above already ties to the gated unfused path
    ma, mr = errors(f64(out2), np.concatenate(refs))
    print(f"swa_prefill_qrope {model}: bitwise equal to RoPE + prefill; bf16-in max_abs={gma:.2e} "
          f"mean_rel={gmr:.2e}; chain max_abs={ma:.2e} mean_rel={mr:.2e}")
    # V read in place: the RoPE call writes K only and the prefill takes v
    # itself as its V staging (the same layout): same output and ring bytes,
    # and held to the oracle on its own
    kst3, _, kring3, vring3, out3 = run_swa_prefill_qrope(batch, v_in_place=True)
    assert torch.equal(kst3.cpu(), kst.cpu())
    assert torch.equal(kring3.cpu(), kring.cpu()) and torch.equal(vring3.cpu(), vring.cpu())
    assert torch.equal(out3.cpu(), out.cpu()), "prefill with V read in place differs"
    assert_close(f64(out3), ref, what=f"swa_prefill_qrope V in place {model}")


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_swa_decode_qrope_against_raw_chain(model):
    """K/V-only RoPE into the rings, then the decode that rotates q itself in
    fp32: against the oracle fed the raw q rotated in fp64 and the exact ring
    bytes, at the bar, and no less accurate than RoPE to a bf16 q_rot followed
    by hsw_swa_decode on the same rings."""
    note(f"swa_decode_qrope {model}")
    positions = [0, 1, 2, 5, 63, 126, 127, 128, 129, 255, 1000, 196608, 205000, 524287, 524288]
    small = wl.swa_decode_batch(seed=82, n_seqs=len(positions), positions=positions,
                                **wl.model_kw(wl.MODELS[model], "swa"))
    big = wl.swa_decode_batch(seed=83, **wl.model_kw(wl.MODELS[model], "swa"))
    for name, batch in (("small positions", small), ("256 sequences", big)):
        shape = batch["shape"]
        S = batch["pos"].shape[0]
        kring, vring = dev(batch["kring"]), dev(batch["vring"])
        hsw.hsw_rope_partial_kv_write(shape, S, None, dev(batch["k"]), dev(batch["v"]), dev(batch["pos"]),
                                      dev(batch["seq"]), RING, kring, vring, S, None, None)
        out = torch.full((S, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
        hsw.hsw_swa_decode_qrope(shape, S, dev(batch["pos"]), dev(batch["q"]), kring, vring,
                                 dev(batch["sinks"]), out)
        # the unfused path on the same rings (RoPE of q only through a scratch K/V destination)
        q_rot = torch.empty_like(dev(batch["q"]))
        kd, vd = torch.empty_like(dev(batch["k"])), torch.empty_like(dev(batch["v"]))
        hsw.hsw_rope_partial_kv_write(shape, S, dev(batch["q"]), dev(batch["k"]), dev(batch["v"]),
                                      dev(batch["pos"]), None, STAGING, kd, vd, S, None, q_rot)
        out_u = torch.empty_like(out)
        hsw.hsw_swa_decode(shape, S, dev(batch["pos"]), q_rot, kring, vring, dev(batch["sinks"]), out_u)
        torch.cuda.synchronize()
        P = batch["pos"].numpy()
        ref = oracle.ring_decode(oracle.rope(f64(batch["q"]), P, shape.rope_theta), P, f64(kring), f64(vring),
                                 sinks=f64(batch["sinks"]), **shape_kw(shape))
        ma, mr = assert_close(f64(out), ref, what=f"swa_decode_qrope {model} {name}")
        mau, mru = errors(f64(out_u), ref)
        print(f"swa_decode_qrope {model} {name}: max_abs={ma:.2e} mean_rel={mr:.2e} "
              f"(bf16 q_rot path: max_abs={mau:.2e} mean_rel={mru:.2e})")
        assert mr <= mru * 1.02, "fp32 rotated q should not be less accurate than a bf16 q_rot"


def run_full_prefill_qrope(batch, kpool, vpool):
    """K/V-only RoPE into the pool, then the chunked prefill that rotates q itself."""
    shape = batch["shape"]
    T = batch["q"].shape[0]
    S = batch["start_pos"].shape[0]
    rows = kpool.shape[0]
    hsw.hsw_rope_partial_kv_write(shape, T, None, dev(batch["k"]), dev(batch["v"]), dev(batch["pos"]),
                                  dev(batch["seq"]), POOL, kpool, vpool, rows, dev(batch["seq_base"]), None)
    lens = batch["cu_seqlens"][1:] - batch["cu_seqlens"][:-1]
    out = torch.full((T, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    hsw.hsw_full_prefill_chunk_qrope(shape, S, int(lens.max()), dev(batch["cu_seqlens"]), dev(batch["start_pos"]),
                                     dev(batch["seq_base"]), dev(batch["q"]), kpool, vpool, rows, None, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("model", ["flash", "pro"])
@pytest.mark.parametrize("case", ["ragged", "large_v", "8192_after_131072"])
def test_full_prefill_qrope_bitwise_equals_rope_then_prefill(case, model):
    """The fused chunked prefill rotates q with the RoPE call's arithmetic and
    stores it as bf16 in the same registers the unfused kernel loads q_rot
    into, so its output is byte-identical to RoPE then hsw_full_prefill_chunk
    over ragged chunks and at the full size, where every output row is
    compared; the fused rows are also held to the oracle fed the unfused
    call's q_rot and pool rows."""
    note(f"full_prefill_qrope bitwise {case} {model}")
    kw = wl.model_kw(wl.MODELS[model], "full")
    if case in ("ragged", "large_v"):
        batch = wl.full_prefill_batch(seed=73, n_seqs=4, seqlens=(300, 77, 129, 1),
                                      start_pos=(3000, 100, 0, 40000), **kw)
        if case == "large_v":
            # out-of-fp16-range values in a late chunk of sequence 0 and in
            # the first chunk of sequence 2: their query blocks take the
            # kernel's general path, fused or not
            base = batch["seq_base"].tolist()
            vp = batch["vpool"].float()
            vp[base[0] + 2500] *= 2.0e5
            vp[base[2] + 10] *= -3.0e5
            batch["vpool"] = vp.to(torch.bfloat16)
    else:
        batch = wl.full_prefill_batch(seed=5, device=DEV, **kw)
    kpool0, vpool0 = dev(batch["kpool"]).clone(), dev(batch["vpool"]).clone()
    q_rot, kpool, vpool, out = run_full_prefill(batch)
    out2 = run_full_prefill_qrope(batch, kpool0, vpool0)
    assert torch.equal(kpool0, kpool) and torch.equal(vpool0, vpool)
    assert torch.equal(out2, out), "fused chunked prefill differs from RoPE + prefill"
    # gate: the fused output against the oracle fed the unfused call's q_rot
    # and pool rows (all rows of the ragged chunks; 256 rows of the full one,
    # drawn apart from the unfused test's sample)
    cu = batch["cu_seqlens"].tolist()
    if case != "8192_after_131072":
        rows = [np.arange(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]
    else:
        rows = [sampled_chunk_rows(8192, seed=6)]
    idx, ref = oracle_full_prefill(batch, q_rot, kpool, vpool, rows)
    bar = dict(max_abs=2e-2 * float(np.abs(ref).max())) if case == "large_v" else {}
    ma, mr = assert_close(f64(out2[torch.from_numpy(idx).to(out2.device)]), ref,
                          what=f"full_prefill_qrope {case} {model}", **bar)
    print(f"full_prefill_qrope {case} {model}: bitwise equal to RoPE + prefill over {out.shape[0]} rows; "
          f"{len(idx)} rows against the oracle: max_abs={ma:.2e} mean_rel={mr:.2e}")


@pytest.mark.parametrize("model", ["flash", "pro"])
@pytest.mark.parametrize("case", ["small", "64_seqs"])
def test_full_decode_qrope_against_raw_chain(case, model):
    """K/V-only RoPE into the pool, then the split-K decode that rotates q
    itself in fp32: against the oracle fed the raw q rotated in fp64 and the
    exact pool bytes, at the bar, and no less accurate than RoPE to a bf16
    q_rot followed by hsw_full_decode_splitk on the same pool."""
    note(f"full_decode_qrope {case} {model}")
    kw = wl.model_kw(wl.MODELS[model], "full")
    if case == "small":
        lengths = [1, 2, 127, 2047, 2048, 2049, 9000, 4097]
        batch = wl.full_decode_batch(seed=62, n_seqs=len(lengths), lengths=lengths, with_sinks=True, **kw)
        seqs, chunk = list(range(len(lengths))), 128
    else:
        batch = wl.full_decode_batch(seed=4, device=DEV, **kw)
        seqs, chunk = c4_sequences(batch["ctx_len"].numpy(), 16, seed=5), 2048
    shape = batch["shape"]
    S = batch["ctx_len"].shape[0]
    sinks = dev(batch.get("sinks"))
    kpool, vpool = dev(batch["kpool"]), dev(batch["vpool"])
    rows = kpool.shape[0]
    hsw.hsw_rope_partial_kv_write(shape, S, None, dev(batch["k"]), dev(batch["v"]), dev(batch["pos"]),
                                  dev(batch["seq"]), POOL, kpool, vpool, rows, dev(batch["seq_base"]), None)
    max_ctx = int(batch["ctx_len"].max())
    wsb = hsw.hsw_full_decode_workspace_bytes(shape, S, max_ctx, chunk)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=DEV)
    out = torch.full((S, shape.n_q_heads, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    hsw.hsw_full_decode_splitk_qrope(shape, S, max_ctx, dev(batch["ctx_len"]), dev(batch["seq_base"]),
                                     dev(batch["q"]), kpool, vpool, rows, sinks, chunk, ws, wsb, out)
    # the unfused path on the same pool (RoPE of q only through a scratch K/V destination)
    q_rot = torch.empty_like(dev(batch["q"]))
    kd, vd = torch.empty_like(dev(batch["k"])), torch.empty_like(dev(batch["v"]))
    hsw.hsw_rope_partial_kv_write(shape, S, dev(batch["q"]), dev(batch["k"]), dev(batch["v"]), dev(batch["pos"]),
                                  None, STAGING, kd, vd, S, None, q_rot)
    out_u = torch.empty_like(out)
    hsw.hsw_full_decode_splitk(shape, S, max_ctx, dev(batch["ctx_len"]), dev(batch["seq_base"]), q_rot,
                               kpool, vpool, rows, sinks, chunk, ws, wsb, out_u)
    torch.cuda.synchronize()
    q_raw = batch["q"].cpu()[seqs]
    qr = oracle.rope(f64(q_raw), batch["pos"].cpu().numpy()[seqs], shape.rope_theta)
    Ls = batch["ctx_len"].tolist()
    base = batch["seq_base"].tolist()
    refs = []
    for i, s in enumerate(seqs):
        k = f64(kpool[base[s]:base[s] + Ls[s]])
        v = f64(vpool[base[s]:base[s] + Ls[s]])
        refs.append(oracle.attn_linear(qr[i:i + 1], [Ls[s] - 1], k, v, 0, window=0,
                                       sinks=None if sinks is None else f64(sinks), **shape_kw(shape))[0])
    ref = np.stack(refs)
    ma, mr = assert_close(f64(out[seqs]), ref, what=f"full_decode_qrope {case} {model}")
    mau, mru = errors(f64(out_u[seqs]), ref)
    print(f"full_decode_qrope {case} {model}: max_abs={ma:.2e} mean_rel={mr:.2e} "
          f"(bf16 q_rot path: max_abs={mau:.2e} mean_rel={mru:.2e})")
    assert mr <= mru * 1.05, "fp32 rotated q should not be less accurate than a bf16 q_rot"
