"""Thin ctypes binding of libhsw.so (include/hsw.h).

Argument marshalling only: every function takes torch tensors for device
memory, passes their data pointers and the current HIP stream to the C entry
point of the same name, and raises HswError on a non-zero status.  All
arithmetic happens in the library's kernels; there is no CPU fallback, and
importing this module fails loudly if the library has not been built.

The library is libhsw.so, or libhsw_checked.so (device-resident arguments
checked on the device) when the environment sets HSW_CHECK_DEVICE=1;
load_library() binds a second copy of these functions to another build in
the same process.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
RELEASE_LIB_PATH = os.path.join(HERE, "libhsw.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libhsw_checked.so")
# load_library() sets _LIB_OVERRIDE on a fresh copy of this module before
# running it
LIB_PATH = (globals().get("_LIB_OVERRIDE")
            or (CHECKED_LIB_PATH if os.environ.get("HSW_CHECK_DEVICE") == "1" else RELEASE_LIB_PATH))

HSW_BF16, HSW_F32 = 0, 1
HSW_DST_RING, HSW_DST_POOL, HSW_DST_STAGING = 0, 1, 2
STATUS = {0: "HSW_OK", 1: "HSW_E_NULL", 2: "HSW_E_SHAPE", 3: "HSW_E_ALIGN", 4: "HSW_E_DTYPE",
          5: "HSW_E_WORKSPACE", 6: "HSW_E_LAUNCH", 7: "HSW_E_CAPACITY", 8: "HSW_E_STALE",
          9: "HSW_E_DEVICE_INPUT"}
HSW_DEV = {0: "OK", 1: "POSITION", 2: "CU_SEQLENS", 3: "POOL_RANGE", 4: "RING_SEQ", 5: "CTX_LEN", 6: "ORDER",
           7: "DST_RANGE"}


class HswError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({detail})")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("value_scale", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class KvmConfig(ctypes.Structure):
    _fields_ = [("n_swa_layers", ctypes.c_int32), ("swa_kv_heads", ctypes.c_int32),
                ("window", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("ring_seqs", ctypes.c_int32),
                ("pool_rows", ctypes.c_int64), ("max_snapshots", ctypes.c_int32)]


_DT = {torch.bfloat16: HSW_BF16, torch.float32: HSW_F32}


def make_shape(s) -> AttnShape:
    """From any object with the fields of workloads.Shape."""
    return AttnShape(s.n_q_heads, s.n_kv_heads, s.d_qk, s.d_v, s.rope_dim, s.window,
                     s.softmax_scale, s.value_scale, s.rope_theta, _DT[s.dtype], _DT[s.out_dtype])


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m hybrid_sliding_window_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SH = ctypes.POINTER(AttnShape)
    lib.hsw_status_str.restype = ctypes.c_char_p
    lib.hsw_status_str.argtypes = [I32]
    lib.hsw_last_error.restype = ctypes.c_char_p
    lib.hsw_version.restype = ctypes.c_char_p
    lib.hsw_device_checks_enabled.restype = I32
    lib.hsw_device_check_status.argtypes = [P, ctypes.POINTER(I32), ctypes.POINTER(I64)]
    lib.hsw_device_check_status.restype = I32
    lib.hsw_rope_partial_kv_write.argtypes = [SH, I64, P, P, P, P, P, I32, P, P, I64, P, P, P, P]
    lib.hsw_swa_prefill.argtypes = [SH, I32, I64, P, P, P, P, P, P, P, P, P, P]
    lib.hsw_swa_decode.argtypes = [SH, I32, P, P, P, P, P, P, P]
    lib.hsw_swa_prefill_qrope.argtypes = [SH, I32, I64, P, P, P, P, P, P, P, P, P, P]
    lib.hsw_swa_decode_qrope.argtypes = [SH, I32, P, P, P, P, P, P, P]
    lib.hsw_full_decode_workspace_bytes.argtypes = [SH, I32, I64, I32]
    lib.hsw_full_decode_workspace_bytes.restype = SZ
    lib.hsw_full_decode_splitk.argtypes = [SH, I32, I64, P, P, P, P, P, I64, P, I32, P, SZ, P, P]
    lib.hsw_full_prefill_chunk.argtypes = [SH, I32, I64, P, P, P, P, P, P, I64, P, P, P]
    lib.hsw_full_prefill_chunk_qrope.argtypes = [SH, I32, I64, P, P, P, P, P, P, I64, P, P, P]
    lib.hsw_full_decode_splitk_qrope.argtypes = [SH, I32, I64, P, P, P, P, P, I64, P, I32, P, SZ, P, P]
    lib.hsw_full_decode_splitk_noalloc.argtypes = [SH, I32, I64, P, P, P, P, P, I64, P, I32, P, P]
    lib.hsw_kv_bytes.argtypes = [I32, I64, I64, I32, I32, I32, I32, I32, I32]
    lib.hsw_vit_layout.argtypes = [I32, I32, P, P, P]
    lib.hsw_vit_rope_2d.argtypes = [SH, I64, P, P, P, P, P, P, P]
    lib.hsw_vit_attention.argtypes = [SH, I32, I64, P, P, I32, P, P, P, P, P, P]
    lib.hsw_vit_window_attention_rope.argtypes = [SH, I32, I64, P, P, I32, P, P, P, P, P, P, P, P]
    lib.hsw_kv_bytes.restype = I64
    KC = ctypes.POINTER(KvmConfig)
    PI32, PI64, PP = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(P)
    lib.hsw_kvm_snapshot_bytes.argtypes = [KC]
    lib.hsw_kvm_snapshot_bytes.restype = SZ
    lib.hsw_kvm_create.argtypes = [KC, PP, PP, P, SZ, PP]
    lib.hsw_kvm_destroy.argtypes = [P]
    lib.hsw_kvm_destroy.restype = None
    lib.hsw_kvm_admit.argtypes = [P, I64, PI32, PI64]
    lib.hsw_kvm_release.argtypes = [P, I32]
    lib.hsw_kvm_append.argtypes = [P, I32, PI32, I64, PI64]
    lib.hsw_kvm_truncate.argtypes = [P, I32, I64]
    lib.hsw_kvm_info.argtypes = [P, I32, PI64, PI64, PI64]
    lib.hsw_kvm_free_space.argtypes = [P, PI32, PI64, PI32]
    lib.hsw_kvm_snapshot.argtypes = [P, I32, PI32, P]
    lib.hsw_kvm_restore.argtypes = [P, I32, P]
    lib.hsw_kvm_drop_snapshot.argtypes = [P, I32]
    lib.hsw_kvm_window_safe_length.argtypes = [P, I32, PI32, I64, PI32]
    lib.hsw_kvm_window_safe_length.restype = I64
    for f in ("hsw_kvm_create", "hsw_kvm_admit", "hsw_kvm_release", "hsw_kvm_append", "hsw_kvm_truncate",
              "hsw_kvm_info", "hsw_kvm_free_space", "hsw_kvm_snapshot", "hsw_kvm_restore",
              "hsw_kvm_drop_snapshot"):
        getattr(lib, f).restype = I32
    for f in ("hsw_rope_partial_kv_write", "hsw_swa_prefill", "hsw_swa_decode", "hsw_swa_prefill_qrope",
              "hsw_swa_decode_qrope", "hsw_full_decode_splitk", "hsw_full_decode_splitk_noalloc",
              "hsw_full_prefill_chunk",
              "hsw_full_decode_splitk_qrope", "hsw_full_prefill_chunk_qrope", "hsw_vit_layout",
              "hsw_vit_rope_2d", "hsw_vit_attention", "hsw_vit_window_attention_rope"):
        getattr(lib, f).restype = I32
    return lib


lib = _load()

EXPORTED = ("hsw_status_str", "hsw_last_error", "hsw_version", "hsw_device_checks_enabled",
            "hsw_device_check_status", "hsw_rope_partial_kv_write",
            "hsw_swa_prefill", "hsw_swa_decode", "hsw_swa_prefill_qrope", "hsw_swa_decode_qrope",
            "hsw_full_decode_workspace_bytes",
            "hsw_full_decode_splitk", "hsw_full_decode_splitk_noalloc", "hsw_full_prefill_chunk",
            "hsw_full_decode_splitk_qrope",
            "hsw_full_prefill_chunk_qrope", "hsw_kv_bytes",
            "hsw_kvm_snapshot_bytes", "hsw_kvm_create", "hsw_kvm_destroy", "hsw_kvm_admit", "hsw_kvm_release",
            "hsw_kvm_append", "hsw_kvm_truncate", "hsw_kvm_info", "hsw_kvm_free_space", "hsw_kvm_snapshot",
            "hsw_kvm_restore", "hsw_kvm_drop_snapshot", "hsw_kvm_window_safe_length",
            "hsw_vit_layout", "hsw_vit_rope_2d", "hsw_vit_attention", "hsw_vit_window_attention_rope")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(rc: int, what: str):
    if rc != 0:
        raise HswError(rc, what, lib.hsw_last_error().decode())


def _sh(shape):
    return ctypes.byref(shape if isinstance(shape, AttnShape) else make_shape(shape))


def hsw_rope_partial_kv_write(shape, n_tokens, q, k, v, pos, seq, dst_kind, k_dst, v_dst,
                              dst_capacity, seq_base, q_rot, dst_index_out=None, stream=None):
    _check(lib.hsw_rope_partial_kv_write(_sh(shape), int(n_tokens), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(pos), _ptr(seq), int(dst_kind), _ptr(k_dst),
                                         _ptr(v_dst), int(dst_capacity), _ptr(seq_base),
                                         _ptr(q_rot), _ptr(dst_index_out), _stream(stream)),
           "hsw_rope_partial_kv_write")


def hsw_swa_prefill(shape, n_seqs, max_seqlen, cu_seqlens, start_pos, q_rot, k_stage, v_stage,
                    k_ring, v_ring, sinks, out, stream=None):
    _check(lib.hsw_swa_prefill(_sh(shape), int(n_seqs), int(max_seqlen), _ptr(cu_seqlens),
                               _ptr(start_pos), _ptr(q_rot), _ptr(k_stage), _ptr(v_stage),
                               _ptr(k_ring), _ptr(v_ring), _ptr(sinks), _ptr(out), _stream(stream)),
           "hsw_swa_prefill")


def hsw_swa_decode(shape, n_seqs, pos, q_rot, k_ring, v_ring, sinks, out, stream=None):
    _check(lib.hsw_swa_decode(_sh(shape), int(n_seqs), _ptr(pos), _ptr(q_rot), _ptr(k_ring),
                              _ptr(v_ring), _ptr(sinks), _ptr(out), _stream(stream)),
           "hsw_swa_decode")


def hsw_swa_prefill_qrope(shape, n_seqs, max_seqlen, cu_seqlens, start_pos, q, k_stage, v_stage,
                          k_ring, v_ring, sinks, out, stream=None):
    _check(lib.hsw_swa_prefill_qrope(_sh(shape), int(n_seqs), int(max_seqlen), _ptr(cu_seqlens),
                                     _ptr(start_pos), _ptr(q), _ptr(k_stage), _ptr(v_stage),
                                     _ptr(k_ring), _ptr(v_ring), _ptr(sinks), _ptr(out), _stream(stream)),
           "hsw_swa_prefill_qrope")


def hsw_swa_decode_qrope(shape, n_seqs, pos, q, k_ring, v_ring, sinks, out, stream=None):
    _check(lib.hsw_swa_decode_qrope(_sh(shape), int(n_seqs), _ptr(pos), _ptr(q), _ptr(k_ring),
                                    _ptr(v_ring), _ptr(sinks), _ptr(out), _stream(stream)),
           "hsw_swa_decode_qrope")


def hsw_full_decode_workspace_bytes(shape, n_seqs, max_ctx, chunk) -> int:
    return int(lib.hsw_full_decode_workspace_bytes(_sh(shape), int(n_seqs), int(max_ctx), int(chunk)))


def hsw_full_decode_splitk(shape, n_seqs, max_ctx, ctx_len, seq_base, q_rot, k_pool, v_pool,
                           pool_rows, sinks, chunk, ws, ws_bytes, out, stream=None):
    _check(lib.hsw_full_decode_splitk(_sh(shape), int(n_seqs), int(max_ctx), _ptr(ctx_len),
                                      _ptr(seq_base), _ptr(q_rot), _ptr(k_pool), _ptr(v_pool),
                                      int(pool_rows), _ptr(sinks), int(chunk), _ptr(ws),
                                      int(ws_bytes), _ptr(out), _stream(stream)),
           "hsw_full_decode_splitk")


NOALLOC_SCRATCH_BYTES = 64 << 20   # HSW_NOALLOC_SCRATCH_BYTES


def hsw_full_decode_splitk_noalloc(shape, n_seqs, max_ctx, ctx_len, seq_base, q_rot, k_pool, v_pool,
                                   pool_rows, sinks, chunk, out, stream=None):
    _check(lib.hsw_full_decode_splitk_noalloc(_sh(shape), int(n_seqs), int(max_ctx), _ptr(ctx_len),
                                              _ptr(seq_base), _ptr(q_rot), _ptr(k_pool), _ptr(v_pool),
                                              int(pool_rows), _ptr(sinks), int(chunk), _ptr(out),
                                              _stream(stream)),
           "hsw_full_decode_splitk_noalloc")


def hsw_full_prefill_chunk(shape, n_seqs, max_seqlen, cu_seqlens, start_pos, seq_base, q_rot,
                           k_pool, v_pool, pool_rows, sinks, out, stream=None):
    _check(lib.hsw_full_prefill_chunk(_sh(shape), int(n_seqs), int(max_seqlen), _ptr(cu_seqlens),
                                      _ptr(start_pos), _ptr(seq_base), _ptr(q_rot), _ptr(k_pool),
                                      _ptr(v_pool), int(pool_rows), _ptr(sinks), _ptr(out),
                                      _stream(stream)),
           "hsw_full_prefill_chunk")


def hsw_full_decode_splitk_qrope(shape, n_seqs, max_ctx, ctx_len, seq_base, q, k_pool, v_pool,
                                 pool_rows, sinks, chunk, ws, ws_bytes, out, stream=None):
    _check(lib.hsw_full_decode_splitk_qrope(_sh(shape), int(n_seqs), int(max_ctx), _ptr(ctx_len),
                                            _ptr(seq_base), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                            int(pool_rows), _ptr(sinks), int(chunk), _ptr(ws),
                                            int(ws_bytes), _ptr(out), _stream(stream)),
           "hsw_full_decode_splitk_qrope")


def hsw_full_prefill_chunk_qrope(shape, n_seqs, max_seqlen, cu_seqlens, start_pos, seq_base, q,
                                 k_pool, v_pool, pool_rows, sinks, out, stream=None):
    _check(lib.hsw_full_prefill_chunk_qrope(_sh(shape), int(n_seqs), int(max_seqlen), _ptr(cu_seqlens),
                                            _ptr(start_pos), _ptr(seq_base), _ptr(q), _ptr(k_pool),
                                            _ptr(v_pool), int(pool_rows), _ptr(sinks), _ptr(out),
                                            _stream(stream)),
           "hsw_full_prefill_chunk_qrope")


def hsw_kv_bytes(kind, n_seqs, ctx, window, n_kv_heads, d_qk, d_v_stored, elem_bytes, n_layers) -> int:
    return int(lib.hsw_kv_bytes(int(kind), int(n_seqs), int(ctx), int(window), int(n_kv_heads),
                                int(d_qk), int(d_v_stored), int(elem_bytes), int(n_layers)))


def hsw_version() -> str:
    return lib.hsw_version().decode()


def hsw_device_checks_enabled() -> bool:
    return bool(lib.hsw_device_checks_enabled())


def hsw_device_check_status(stream=None):
    """(status, code, index) of the current device's check flag (the flag is
    cleared when a violation is reported); code -1 in a release build."""
    code, index = ctypes.c_int32(), ctypes.c_int64()
    rc = int(lib.hsw_device_check_status(_stream(stream), ctypes.byref(code), ctypes.byref(index)))
    return rc, code.value, index.value


def load_library(path):
    """A second copy of this binding, on the library at `path` (e.g.
    CHECKED_LIB_PATH), as a module object with the same functions."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(f"{__name__}_{os.path.basename(path)}", __file__)
    mod = importlib.util.module_from_spec(spec)
    mod._LIB_OVERRIDE = path
    spec.loader.exec_module(mod)
    return mod


def hsw_kvm_snapshot_bytes(cfg: KvmConfig) -> int:
    return int(lib.hsw_kvm_snapshot_bytes(ctypes.byref(cfg)))


def _ids(tokens):
    arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
    return arr, len(tokens)


class KvManager:
    """The hsw_kvm_* calls on one handle (marshalling only).  swa_k / swa_v:
    the per-layer ring tensors (device), snap_buf: a device tensor of at least
    max_snapshots * hsw_kvm_snapshot_bytes(cfg) bytes (or None)."""

    def __init__(self, cfg: KvmConfig, swa_k, swa_v, snap_buf=None):
        n = cfg.n_swa_layers
        self.cfg = cfg
        self._keep = (list(swa_k), list(swa_v), snap_buf)   # the tensors outlive the handle
        ks = (ctypes.c_void_p * n)(*[_ptr(t) for t in swa_k])
        vs = (ctypes.c_void_p * n)(*[_ptr(t) for t in swa_v])
        nbytes = 0 if snap_buf is None else snap_buf.numel() * snap_buf.element_size()
        h = ctypes.c_void_p()
        _check(lib.hsw_kvm_create(ctypes.byref(cfg), ks, vs, _ptr(snap_buf), nbytes, ctypes.byref(h)),
               "hsw_kvm_create")
        self.h = h

    def close(self):
        if self.h:
            lib.hsw_kvm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, max_len):
        seq, base = ctypes.c_int32(), ctypes.c_int64()
        _check(lib.hsw_kvm_admit(self.h, int(max_len), ctypes.byref(seq), ctypes.byref(base)), "hsw_kvm_admit")
        return seq.value, base.value

    def release(self, seq):
        _check(lib.hsw_kvm_release(self.h, int(seq)), "hsw_kvm_release")

    def append(self, seq, tokens):
        arr, n = _ids(tokens)
        start = ctypes.c_int64()
        _check(lib.hsw_kvm_append(self.h, int(seq), arr, n, ctypes.byref(start)), "hsw_kvm_append")
        return start.value

    def truncate(self, seq, new_len):
        _check(lib.hsw_kvm_truncate(self.h, int(seq), int(new_len)), "hsw_kvm_truncate")

    def info(self, seq):
        ln, base, mx = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib.hsw_kvm_info(self.h, int(seq), ctypes.byref(ln), ctypes.byref(base), ctypes.byref(mx)),
               "hsw_kvm_info")
        return ln.value, base.value, mx.value

    def free_space(self):
        r, run, sn = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib.hsw_kvm_free_space(self.h, ctypes.byref(r), ctypes.byref(run), ctypes.byref(sn)),
               "hsw_kvm_free_space")
        return r.value, run.value, sn.value

    def snapshot(self, seq, stream=None):
        snap = ctypes.c_int32()
        _check(lib.hsw_kvm_snapshot(self.h, int(seq), ctypes.byref(snap), _stream(stream)), "hsw_kvm_snapshot")
        return snap.value

    def restore(self, snap, stream=None):
        _check(lib.hsw_kvm_restore(self.h, int(snap), _stream(stream)), "hsw_kvm_restore")

    def drop_snapshot(self, snap):
        _check(lib.hsw_kvm_drop_snapshot(self.h, int(snap)), "hsw_kvm_drop_snapshot")

    def window_safe_length(self, seq, tokens):
        arr, n = _ids(tokens)
        snap = ctypes.c_int32()
        L = int(lib.hsw_kvm_window_safe_length(self.h, int(seq), arr, n, ctypes.byref(snap)))
        if L < 0:
            raise HswError(2, "hsw_kvm_window_safe_length", lib.hsw_last_error().decode())
        return L, snap.value


# ------------------------------------------------------------------ vision
def hsw_vit_layout(h, w):
    """(row, col, col_order) int32 numpy arrays of an h x w patch grid in
    merge-unit order (host arithmetic in the library)."""
    import numpy as np
    n = int(h) * int(w)
    row, col, co = (np.empty(max(n, 0), np.int32) for _ in range(3))
    _check(lib.hsw_vit_layout(int(h), int(w), row.ctypes.data_as(ctypes.c_void_p), col.ctypes.data_as(ctypes.c_void_p),
                              co.ctypes.data_as(ctypes.c_void_p)), "hsw_vit_layout")
    return row, col, co


def hsw_vit_rope_2d(shape, n_tokens, q, k, row, col, q_out, k_out, stream=None):
    _check(lib.hsw_vit_rope_2d(_sh(shape), int(n_tokens), _ptr(q), _ptr(k), _ptr(row), _ptr(col),
                               _ptr(q_out), _ptr(k_out), _stream(stream)), "hsw_vit_rope_2d")


def hsw_vit_attention(shape, n_images, max_len, cu_seqlens, order, sink_key, q, k, v, sinks, out,
                      stream=None):
    _check(lib.hsw_vit_attention(_sh(shape), int(n_images), int(max_len), _ptr(cu_seqlens), _ptr(order),
                                 int(sink_key), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out),
                                 _stream(stream)), "hsw_vit_attention")


def hsw_vit_window_attention_rope(shape, n_images, max_len, cu_seqlens, order, sink_key, row, col, q, k, v,
                                  sinks, out, stream=None):
    _check(lib.hsw_vit_window_attention_rope(_sh(shape), int(n_images), int(max_len), _ptr(cu_seqlens),
                                             _ptr(order), int(sink_key), _ptr(row), _ptr(col), _ptr(q), _ptr(k),
                                             _ptr(v), _ptr(sinks), _ptr(out), _stream(stream)),
           "hsw_vit_window_attention_rope")
