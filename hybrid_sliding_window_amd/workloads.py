"""Seeded synthetic workloads for the attention core (shapes, seeds and value
distributions only -- none of the method's arithmetic lives here).

This is the one module that both the HIP path's tests/benchmark and the fp64
oracle's inputs come from.  It imports torch and nothing of the library.

Shapes follow the pages: MiMo-V2.6-Flash windowed layers have 8 KV heads and
full layers 4 (colibri "What the engine implements"), q/k heads are 192 wide
and v heads 128, the window/ring is 128 positions, 48 layers of which 39 are
windowed (colibri, model table).  The query head count of Flash is not printed
on the pages; 64 is used.  MiMo-V2.6-Pro has 70 layers, 60 windowed + 10 full
(colibri, model table), 128 query and 8 KV heads, one KV head per rank on both
layer kinds at TP8 (gaudi-cookbook, "MiMo-V2.6-Pro"), and value scale 0.612
against Flash's 0.707 (colibri, "What the engine implements").  Prefill
chunks of 8192 tokens and contexts up to 512K come from the gaudi-cookbook
page ("At a glance", "Tiled global-attention prefill").

Recipes (every draw comes from a torch.Generator seeded as stated):
  * values: standard normal fp32, rounded to bf16 (round-to-nearest-even) for
    the bf16 workloads; sinks ~ N(1, 0.25) (std 0.25) in fp32;
  * integers (positions, lengths): torch.randint on a CPU generator;
  * the logit-shift workload moves one RoPE pass-through dim (191) of q up by
    38.12 and of k down by 9.09 so scaled logits sit near -25 +- 3 while the
    sinks sit near +1 (gaudi-cookbook "What was built": the sink normally
    takes almost all the attention mass).
"""
from __future__ import annotations

import dataclasses
import math

import torch

D_QK, D_V, ROPE_DIM, WINDOW = 192, 128, 64, 128
THETA_SWA, THETA_FULL = 1.0e4, 1.0e7
VALUE_SCALE_FLASH, VALUE_SCALE_PRO = 0.707, 0.612
SOFTMAX_SCALE = 1.0 / math.sqrt(D_QK)
LOGIT_SHIFT_Q, LOGIT_SHIFT_K = 38.12, 9.09


@dataclasses.dataclass(frozen=True)
class Model:
    """Head counts, value scale and layer mix of one model of the family."""
    name: str
    n_q_heads: int
    swa_kv_heads: int
    full_kv_heads: int
    value_scale: float
    n_layers: int
    n_full: int


FLASH = Model("MiMo-V2.6-Flash", 64, 8, 4, VALUE_SCALE_FLASH, 48, 9)
PRO = Model("MiMo-V2.6-Pro", 128, 8, 8, VALUE_SCALE_PRO, 70, 10)
MODELS = {"flash": FLASH, "pro": PRO}


@dataclasses.dataclass(frozen=True)
class Shape:
    """Per-layer attention shape (mirrors the C struct hsw_attn_shape)."""
    n_q_heads: int
    n_kv_heads: int
    window: int                  # 0 = full attention
    rope_theta: float
    d_qk: int = D_QK
    d_v: int = D_V
    rope_dim: int = ROPE_DIM
    softmax_scale: float = SOFTMAX_SCALE
    value_scale: float = VALUE_SCALE_FLASH
    dtype: torch.dtype = torch.bfloat16
    out_dtype: torch.dtype = torch.bfloat16


def swa_shape(hq=64, hkv=8, dtype=torch.bfloat16, out_dtype=None, value_scale=VALUE_SCALE_FLASH):
    return Shape(hq, hkv, WINDOW, THETA_SWA, dtype=dtype,
                 out_dtype=out_dtype or dtype, value_scale=value_scale)


def full_shape(hq=64, hkv=4, dtype=torch.bfloat16, out_dtype=None, value_scale=VALUE_SCALE_FLASH):
    return Shape(hq, hkv, 0, THETA_FULL, dtype=dtype,
                 out_dtype=out_dtype or dtype, value_scale=value_scale)


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, g: torch.Generator, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """Standard normal fp32 draw, then RNE to `dtype`."""
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


def randn_rows(shape, g: torch.Generator, dtype=torch.bfloat16, device="cpu",
               max_elems=1 << 28) -> torch.Tensor:
    """randn() drawn slice by slice along the first dimension (at most
    max_elems per slice), so a pool far larger than free memory / 3 can be
    filled without one fp32 temporary of its whole size.  Deterministic for a
    given generator state and max_elems."""
    out = torch.empty(tuple(shape), dtype=dtype, device=device)
    per_row = max(1, math.prod(shape[1:]))
    step = max(1, max_elems // per_row)
    for r0 in range(0, shape[0], step):
        r1 = min(shape[0], r0 + step)
        out[r0:r1] = randn((r1 - r0, *shape[1:]), g, dtype, device)
    return out


def sinks(n_q_heads: int, g: torch.Generator) -> torch.Tensor:
    return (1.0 + 0.25 * torch.randn((n_q_heads,), generator=g, dtype=torch.float32))


# --------------------------------------------------------------------------
# Workload 1: one windowed layer in fp32, 1 x 512 tokens, 4/1 heads,
# logits shifted to about -25 so the sink dominates.
# --------------------------------------------------------------------------
def logit_shift_layer(seed=1, n_tok=512, hq=4, hkv=1, dtype=torch.float32, start=0):
    g = gen(seed)
    q = randn((n_tok, hq, D_QK), g, torch.float32)
    k = randn((n_tok, hkv, D_QK), g, torch.float32)
    v = randn((n_tok, hkv, D_V), g, torch.float32)
    q[..., D_QK - 1] += LOGIT_SHIFT_Q
    k[..., D_QK - 1] -= LOGIT_SHIFT_K
    return dict(shape=swa_shape(hq, hkv, dtype=dtype), q=q.to(dtype), k=k.to(dtype),
                v=v.to(dtype), pos=torch.arange(start, start + n_tok, dtype=torch.int64),
                seq=torch.zeros(n_tok, dtype=torch.int32), sinks=sinks(hq, g),
                cu_seqlens=torch.tensor([0, n_tok], dtype=torch.int64),
                start_pos=torch.tensor([start], dtype=torch.int64))


# --------------------------------------------------------------------------
# Workload 2: windowed prefill, S sequences x T tokens from position `start`.
# --------------------------------------------------------------------------
def swa_prefill_batch(seed=2, n_seqs=4, seqlens=(8192,) * 4, start_pos=None, hq=64, hkv=8,
                      dtype=torch.bfloat16, device="cpu", value_scale=VALUE_SCALE_FLASH):
    """q/k/v for a prefill chunk of `n_seqs` sequences (ragged lengths allowed)
    plus, for each sequence, a ring already holding the 127 positions before
    its start (zeros where the position would be < 0 are never read)."""
    assert len(seqlens) == n_seqs
    g = gen(seed)
    start = [0] * n_seqs if start_pos is None else list(start_pos)
    T = int(sum(seqlens))
    gd = gen(seed + 1000, device) if device != "cpu" else g
    q = randn((T, hq, D_QK), gd, dtype, device)
    k = randn((T, hkv, D_QK), gd, dtype, device)
    v = randn((T, hkv, D_V), gd, dtype, device)
    kring = randn((n_seqs, hkv, WINDOW, D_QK), gd, dtype, device)
    vring = randn((n_seqs, hkv, WINDOW, D_V), gd, dtype, device)
    cu = torch.zeros(n_seqs + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0)
    pos = torch.cat([torch.arange(s, s + n, dtype=torch.int64) for s, n in zip(start, seqlens)])
    seq = torch.cat([torch.full((n,), i, dtype=torch.int32) for i, n in enumerate(seqlens)])
    return dict(shape=swa_shape(hq, hkv, dtype=dtype, value_scale=value_scale), q=q, k=k, v=v, kring=kring,
                vring=vring, pos=pos, seq=seq, cu_seqlens=cu,
                start_pos=torch.tensor(start, dtype=torch.int64), sinks=sinks(hq, g))


# --------------------------------------------------------------------------
# Workload 3: windowed decode, S sequences at positions U{lo .. hi}.
# --------------------------------------------------------------------------
def swa_decode_batch(seed=3, n_seqs=256, pos_lo=128, pos_hi=524288, hq=64, hkv=8,
                     dtype=torch.bfloat16, device="cpu", positions=None, value_scale=VALUE_SCALE_FLASH):
    g = gen(seed)
    if positions is None:
        pos = torch.randint(pos_lo, pos_hi + 1, (n_seqs,), generator=g, dtype=torch.int64)
    else:
        pos = torch.as_tensor(positions, dtype=torch.int64)
    s = sinks(hq, g)
    gd = gen(seed + 1000, device) if device != "cpu" else g
    kring = randn((n_seqs, hkv, WINDOW, D_QK), gd, dtype, device)
    vring = randn((n_seqs, hkv, WINDOW, D_V), gd, dtype, device)
    q = randn((n_seqs, hq, D_QK), gd, dtype, device)
    k = randn((n_seqs, hkv, D_QK), gd, dtype, device)
    v = randn((n_seqs, hkv, D_V), gd, dtype, device)
    return dict(shape=swa_shape(hq, hkv, dtype=dtype, value_scale=value_scale), q=q, k=k, v=v, kring=kring,
                vring=vring, pos=pos, seq=torch.arange(n_seqs, dtype=torch.int32), sinks=s)


# --------------------------------------------------------------------------
# Workload 4: full-attention decode over a contiguous pool.
# Sequence s owns rows seq_base[s] .. seq_base[s] + L_s - 1; rows 0..L_s-2
# are prior context, the new token (position L_s - 1) is appended by RoPE.
# --------------------------------------------------------------------------
def full_decode_batch(seed=4, n_seqs=64, len_lo=32768, len_hi=131072, hq=64, hkv=4,
                      dtype=torch.bfloat16, device="cpu", lengths=None, with_sinks=False,
                      value_scale=VALUE_SCALE_FLASH):
    g = gen(seed)
    if lengths is None:
        L = torch.randint(len_lo, len_hi + 1, (n_seqs,), generator=g, dtype=torch.int64)
    else:
        L = torch.as_tensor(lengths, dtype=torch.int64)
    base = torch.zeros(n_seqs, dtype=torch.int64)
    base[1:] = torch.cumsum(L, 0)[:-1]
    rows = int(L.sum())
    s = sinks(hq, g) if with_sinks else None
    gd = gen(seed + 1000, device) if device != "cpu" else g
    kpool = randn((rows, hkv, D_QK), gd, dtype, device)
    vpool = randn((rows, hkv, D_V), gd, dtype, device)
    q = randn((n_seqs, hq, D_QK), gd, dtype, device)
    k = randn((n_seqs, hkv, D_QK), gd, dtype, device)
    v = randn((n_seqs, hkv, D_V), gd, dtype, device)
    return dict(shape=full_shape(hq, hkv, dtype=dtype, value_scale=value_scale), q=q, k=k, v=v, kpool=kpool,
                vpool=vpool, ctx_len=L, seq_base=base, pos=L - 1, seq=torch.arange(n_seqs, dtype=torch.int32),
                sinks=s)


# --------------------------------------------------------------------------
# Workload 5 pieces: full-attention prefill chunk with prior context.
# --------------------------------------------------------------------------
def full_prefill_batch(seed=5, n_seqs=1, seqlens=(8192,), start_pos=(131072,), hq=64, hkv=4,
                       dtype=torch.bfloat16, device="cpu", value_scale=VALUE_SCALE_FLASH):
    """One chunk per sequence: prior rows 0..start-1 in the pool, the chunk's
    own q/k/v at positions start .. start+T-1 (appended by RoPE)."""
    g = gen(seed)
    start = list(start_pos)
    seqlens = list(seqlens)
    L = torch.tensor([s + n for s, n in zip(start, seqlens)], dtype=torch.int64)
    base = torch.zeros(n_seqs, dtype=torch.int64)
    base[1:] = torch.cumsum(L, 0)[:-1]
    rows = int(L.sum())
    T = int(sum(seqlens))
    gd = gen(seed + 1000, device) if device != "cpu" else g
    kpool = randn((rows, hkv, D_QK), gd, dtype, device)
    vpool = randn((rows, hkv, D_V), gd, dtype, device)
    q = randn((T, hq, D_QK), gd, dtype, device)
    k = randn((T, hkv, D_QK), gd, dtype, device)
    v = randn((T, hkv, D_V), gd, dtype, device)
    cu = torch.zeros(n_seqs + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0)
    pos = torch.cat([torch.arange(s, s + n, dtype=torch.int64) for s, n in zip(start, seqlens)])
    seq = torch.cat([torch.full((n,), i, dtype=torch.int32) for i, n in enumerate(seqlens)])
    return dict(shape=full_shape(hq, hkv, dtype=dtype, value_scale=value_scale), q=q, k=k, v=v, kpool=kpool,
                vpool=vpool, cu_seqlens=cu, start_pos=torch.tensor(start, dtype=torch.int64), seq_base=base,
                ctx_len=L, pos=pos, seq=seq)


def model_kw(model: Model, kind: str) -> dict:
    """Head counts and value scale of `model` for a batch generator of layer
    kind "swa" or "full"."""
    hkv = model.swa_kv_heads if kind == "swa" else model.full_kv_heads
    return dict(hq=model.n_q_heads, hkv=hkv, value_scale=model.value_scale)


def hybrid_pattern(seed=5, n_layers=48, n_full=9):
    """hybrid_layer_pattern: 1 = windowed, 0 = full; the full layers' indices
    are the first n_full entries of a seeded permutation of the layers (the
    real pattern is not printed on the pages)."""
    g = gen(seed)
    perm = torch.randperm(n_layers, generator=g)
    pat = [1] * n_layers
    for i in perm[:n_full].tolist():
        pat[i] = 0
    return pat


# ------------------------------------------------------------------ vision
# The vision encoder's attention (colibri "MiMo-V2.6 (Xiaomi)", the "vision"
# entry).  The pages give no head sizes: 16 query / 4 KV heads of width 64
# are used, softmax scale 1/8, RoPE theta 1e4.  Pictures are patch grids with
# even sides (2x2 merge units); the page's own picture gives 252 merged rows,
# i.e. 1008 patches, taken here as a 28 x 36 grid.  The token layout (patch
# coordinates, unit orders) is method arithmetic and is not computed here.
VIT_D, VIT_THETA = 64, 1.0e4
VIT_PAGE_GRID = (28, 36)
VIT_BENCH_GRIDS = ((64, 64),) * 16          # 16 pictures of 896 x 896 px at 14 px patches


def vit_shape(hq=16, hkv=4, window=64):
    return Shape(hq, hkv, window, VIT_THETA, d_qk=VIT_D, d_v=VIT_D, rope_dim=VIT_D,
                 softmax_scale=1.0 / math.sqrt(VIT_D), value_scale=1.0)


def vit_batch(seed=9, grids=(VIT_PAGE_GRID,), hq=16, hkv=4, q_scale=1.0, with_sinks=False, device="cpu"):
    """Pictures packed by token rows: q [T, hq, 64], k, v [T, hkv, 64] bf16
    (q optionally scaled by q_scale before rounding, for peaked attention),
    cu_seqlens int64, the grids, and (with_sinks) sink logits ~ N(1, 0.25)."""
    g = gen(seed)
    lens = [h * w for h, w in grids]
    T = sum(lens)
    cu = torch.zeros(len(lens) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0)
    gd = gen(seed * 1000 + 1, device)
    q = (torch.randn((T, hq, VIT_D), generator=gd, device=device) * q_scale).to(torch.bfloat16)
    k = randn((T, hkv, VIT_D), gd, device=device)
    v = randn((T, hkv, VIT_D), gd, device=device)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, grids=list(grids), lens=lens,
                sinks=sinks(hq, g) if with_sinks else None)
