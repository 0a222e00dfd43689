"""The hybrid step: a driver of the C-ABI calls over the layers of a hybrid
windowed / full-attention stack (argument marshalling only; every step runs in
the library's kernels).

colibri "MiMo-V2.6 (Xiaomi)", "What the engine implements": windowed layers
keep a 128-slot ring per sequence and KV head, full layers keep every
position; gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", "What was built": the
windowed layers carry per-head sinks.  One step serves a prefill chunk and a
batch of decode sequences on every layer:

  windowed layer: RoPE + staging write of the chunk, windowed prefill (keys
                  before the chunk from the chunk sequence's ring, then the
                  ring commit), RoPE + ring write of the decode tokens,
                  windowed decode;
  full layer:     RoPE + pool write of the chunk, chunked full prefill over
                  the pool, RoPE + pool write of the decode tokens, split-K
                  full decode.

With qrope=True the RoPE calls rotate and write K/V only and each attention
call is its *_qrope form, which rotates the raw q itself (no q_rot round trip
through HBM); on windowed layers the chunk's RoPE call writes K alone and the
prefill reads the chunk's V where it is (its layout is the staging one).

step(overlap=True) issues each layer's decode calls on a second stream: the
decode chain (RoPE + decode of the decode tokens, layer after layer) and the
prefill chain (RoPE + prefill of the chunk, layer after layer) share no data
-- disjoint pool rows, rings and outputs -- so the HBM-bound decodes run
beside the compute-bound prefills; each chain keeps its own layer order.

Sizes default to the bench workload: the model's layers (MiMo-V2.6-Flash: 48,
39 windowed + 9 full; MiMo-V2.6-Pro: 70, 60 + 10; the full layers at seeded
indices), an 8192-token chunk at positions 131072..139263 and 128 decode
sequences with contexts U{4096..262144}.  Per-layer q/k/v are generated up
front; the full layers share one pool (each full layer reads the same number
of bytes, and a pool per full layer would exceed one GPU's memory).
"""
from __future__ import annotations

import torch

from . import workloads as wl


class HybridStep:
    def __init__(self, hsw, pattern=None, T=8192, P0=131072, S=128, ctx_lo=4096, ctx_hi=262144, seed=5,
                 device="cuda:0", chunk=2048, model=wl.FLASH, qrope=False):
        self.hsw = hsw
        self.model = model
        self.qrope = qrope
        self.pattern = (list(wl.hybrid_pattern(seed, model.n_layers, model.n_full)) if pattern is None
                        else list(pattern))
        self.T, self.P0, self.S, self.chunk = T, P0, S, chunk
        hq, hs, hf = model.n_q_heads, model.swa_kv_heads, model.full_kv_heads
        self.hq, self.hkv_swa, self.hkv_full = hq, hs, hf
        self.swa = wl.swa_shape(hq, hs, value_scale=model.value_scale)
        self.full = wl.full_shape(hq, hf, value_scale=model.value_scale)
        g = wl.gen(seed)
        self.L = torch.randint(ctx_lo, ctx_hi + 1, (S,), generator=g, dtype=torch.int64)
        gd = wl.gen(seed * 1000, device)
        self.layers = []
        for kind in self.pattern:
            hkv = hs if kind == 1 else hf
            d = dict(qc=wl.randn((T, hq, 192), gd, device=device), kc=wl.randn((T, hkv, 192), gd, device=device),
                     vc=wl.randn((T, hkv, 128), gd, device=device), qd=wl.randn((S, hq, 192), gd, device=device),
                     kd=wl.randn((S, hkv, 192), gd, device=device), vd=wl.randn((S, hkv, 128), gd, device=device))
            if kind == 1:
                # rings: decode sequences 0..S-1, the chunk's sequence at index S
                d["kring"] = wl.randn((S + 1, hs, 128, 192), gd, device=device)
                d["vring"] = wl.randn((S + 1, hs, 128, 128), gd, device=device)
            self.layers.append(d)
        self.sinks = wl.sinks(hq, g).to(device)
        # shared full-attention pool: the chunk sequence at rows [0, P0 + T),
        # then the decode sequences
        base = torch.zeros(S, dtype=torch.int64)
        base[0] = P0 + T
        base[1:] = P0 + T + torch.cumsum(self.L, 0)[:-1]
        self.base_dec = base
        self.rows = int(P0 + T + self.L.sum())
        self.kpool = wl.randn_rows((self.rows, hf, 192), gd, device=device)
        self.vpool = wl.randn_rows((self.rows, hf, 128), gd, device=device)
        self.d_L, self.d_base_dec = self.L.to(device), base.to(device)
        self.d_pos_dec = (self.L - 1).to(device)
        self.d_seq_dec = torch.arange(S, dtype=torch.int32, device=device)
        self.d_pos_c = torch.arange(P0, P0 + T, dtype=torch.int64, device=device)
        self.d_seq_c0 = torch.zeros(T, dtype=torch.int32, device=device)
        self.d_cu = torch.tensor([0, T], dtype=torch.int64, device=device)
        self.d_start = torch.tensor([P0], dtype=torch.int64, device=device)
        self.d_base_c = torch.zeros(1, dtype=torch.int64, device=device)
        bf = torch.bfloat16
        self.q_rot = torch.empty((T, hq, 192), dtype=bf, device=device)
        self.q_rot_d = torch.empty((S, hq, 192), dtype=bf, device=device)
        self.kst = torch.empty((T, hs, 192), dtype=bf, device=device)
        self.vst = torch.empty((T, hs, 128), dtype=bf, device=device)
        self.out = torch.empty((T, hq, 128), dtype=bf, device=device)
        self.out_d = torch.empty((S, hq, 128), dtype=bf, device=device)
        self.max_ctx = int(self.L.max())
        self.wsb = hsw.hsw_full_decode_workspace_bytes(self.full, S, self.max_ctx, chunk)
        self.ws = torch.empty(self.wsb // 4 + 4, dtype=torch.float32, device=device)

    def calls(self, li, stream=None, qrope=None, dstream=None):
        """The four calls of layer li as (name, thunk) pairs, in order
        (qrope: override the instance's choice of fused q-RoPE; dstream: the
        stream of the two decode calls, default `stream`)."""
        if dstream is not None:
            pre = self.calls(li, stream, qrope)[:2]
            return pre + self.calls(li, dstream, qrope)[2:]
        if self.qrope if qrope is None else qrope:
            return self._calls_qrope(li, stream)
        h, d, T, S = self.hsw, self.layers[li], self.T, self.S
        if self.pattern[li] == 1:
            swa = self.swa
            return [
                ("rope", lambda: h.hsw_rope_partial_kv_write(swa, T, d["qc"], d["kc"], d["vc"], self.d_pos_c, None,
                                                             h.HSW_DST_STAGING, self.kst, self.vst, T, None,
                                                             self.q_rot, None, stream)),
                ("swa_prefill", lambda: h.hsw_swa_prefill(swa, 1, T, self.d_cu, self.d_start, self.q_rot, self.kst,
                                                          self.vst, d["kring"][S:], d["vring"][S:], self.sinks,
                                                          self.out, stream)),
                ("rope", lambda: h.hsw_rope_partial_kv_write(swa, S, d["qd"], d["kd"], d["vd"], self.d_pos_dec,
                                                             self.d_seq_dec, h.HSW_DST_RING, d["kring"], d["vring"],
                                                             S + 1, None, self.q_rot_d, None, stream)),
                ("swa_decode", lambda: h.hsw_swa_decode(swa, S, self.d_pos_dec, self.q_rot_d, d["kring"], d["vring"],
                                                        self.sinks, self.out_d, stream)),
            ]
        full = self.full
        return [
            ("rope", lambda: h.hsw_rope_partial_kv_write(full, T, d["qc"], d["kc"], d["vc"], self.d_pos_c,
                                                         self.d_seq_c0, h.HSW_DST_POOL, self.kpool, self.vpool,
                                                         self.rows, self.d_base_c, self.q_rot, None, stream)),
            ("full_prefill", lambda: h.hsw_full_prefill_chunk(full, 1, T, self.d_cu, self.d_start, self.d_base_c,
                                                              self.q_rot, self.kpool, self.vpool, self.rows, None,
                                                              self.out, stream)),
            ("rope", lambda: h.hsw_rope_partial_kv_write(full, S, d["qd"], d["kd"], d["vd"], self.d_pos_dec,
                                                         self.d_seq_dec, h.HSW_DST_POOL, self.kpool, self.vpool,
                                                         self.rows, self.d_base_dec, self.q_rot_d, None, stream)),
            ("full_decode", lambda: h.hsw_full_decode_splitk(full, S, self.max_ctx, self.d_L, self.d_base_dec,
                                                             self.q_rot_d, self.kpool, self.vpool, self.rows, None,
                                                             self.chunk, self.ws, self.wsb, self.out_d, stream)),
        ]

    def _calls_qrope(self, li, stream):
        h, d, T, S = self.hsw, self.layers[li], self.T, self.S
        if self.pattern[li] == 1:
            swa = self.swa
            return [
                # K only into staging: the prefill reads the chunk's V in place
                ("rope", lambda: h.hsw_rope_partial_kv_write(swa, T, None, d["kc"], None, self.d_pos_c, None,
                                                             h.HSW_DST_STAGING, self.kst, None, T, None, None,
                                                             None, stream)),
                ("swa_prefill", lambda: h.hsw_swa_prefill_qrope(swa, 1, T, self.d_cu, self.d_start, d["qc"],
                                                                self.kst, d["vc"], d["kring"][S:], d["vring"][S:],
                                                                self.sinks, self.out, stream)),
                ("rope", lambda: h.hsw_rope_partial_kv_write(swa, S, None, d["kd"], d["vd"], self.d_pos_dec,
                                                             self.d_seq_dec, h.HSW_DST_RING, d["kring"], d["vring"],
                                                             S + 1, None, None, None, stream)),
                ("swa_decode", lambda: h.hsw_swa_decode_qrope(swa, S, self.d_pos_dec, d["qd"], d["kring"],
                                                              d["vring"], self.sinks, self.out_d, stream)),
            ]
        full = self.full
        return [
            ("rope", lambda: h.hsw_rope_partial_kv_write(full, T, None, d["kc"], d["vc"], self.d_pos_c,
                                                         self.d_seq_c0, h.HSW_DST_POOL, self.kpool, self.vpool,
                                                         self.rows, self.d_base_c, None, None, stream)),
            ("full_prefill", lambda: h.hsw_full_prefill_chunk_qrope(full, 1, T, self.d_cu, self.d_start,
                                                                    self.d_base_c, d["qc"], self.kpool, self.vpool,
                                                                    self.rows, None, self.out, stream)),
            ("rope", lambda: h.hsw_rope_partial_kv_write(full, S, None, d["kd"], d["vd"], self.d_pos_dec,
                                                         self.d_seq_dec, h.HSW_DST_POOL, self.kpool, self.vpool,
                                                         self.rows, self.d_base_dec, None, None, stream)),
            ("full_decode", lambda: h.hsw_full_decode_splitk_qrope(full, S, self.max_ctx, self.d_L,
                                                                   self.d_base_dec, d["qd"], self.kpool, self.vpool,
                                                                   self.rows, None, self.chunk, self.ws, self.wsb,
                                                                   self.out_d, stream)),
        ]

    def step(self, stream=None, timer=None, overlap=False):
        """Every layer in order.  timer: a list that receives (name, start
        event, end event) per call.  overlap: decode calls on a second stream
        (joined back into `stream` at the end)."""
        if overlap:
            main = stream if stream is not None else torch.cuda.current_stream()
            if getattr(self, "_dstream", None) is None:
                self._dstream = torch.cuda.Stream(device=main.device)   # default priority
            ds = self._dstream
            ds.wait_stream(main)
            for li in range(len(self.pattern)):
                for name, fn in self.calls(li, main, dstream=ds):
                    fn()
            main.wait_stream(ds)
            return
        for li in range(len(self.pattern)):
            for name, fn in self.calls(li, stream):
                if timer is None:
                    fn()
                else:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    timer.append((name, e0, e1))

    @property
    def pool_gb(self):
        return self.rows * self.hkv_full * 320 * 2 / 1e9
