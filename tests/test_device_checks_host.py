"""The device-argument contract of the checked build, on the CPU.

hybrid_sliding_window_amd/csrc/dev_check.h holds one predicate per checked
element, which the check kernel of libhsw_checked.so runs on the device.  The
header is plain C++ as well: this test builds it with g++ into a small host
library and runs every rule of include/hsw.h's "Device-resident argument
checks" on hand-made arrays -- a valid case per call, then each violation at
a chosen element, which must give that rule's code at that element.  The
release library's status call is checked too: it reports "not checked"
without touching a GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_sliding_window_amd", "csrc")

OK, POSITION, CU_SEQLENS, POOL_RANGE, RING_SEQ, CTX_LEN, ORDER, DST_RANGE = range(8)
ROPE, SWA_PREFILL, SWA_DECODE, FULL_DECODE, FULL_PREFILL, VIT = range(6)
RING, POOL, STAGING = 0, 1, 2

DRIVER = r"""
#include "dev_check.h"
extern "C" int32_t first_violation(const hsw::devcheck::Inputs *in, int64_t *where) {
    for (int64_t i = 0; i < in->n; ++i) {
        int32_t c = hsw::devcheck::check_element(*in, i);
        if (c) { *where = i; return c; }
    }
    *where = -1;
    return 0;
}
"""


class Inputs(ctypes.Structure):
    P = ctypes.c_void_p
    _fields_ = [("call", ctypes.c_int32), ("dst_kind", ctypes.c_int32), ("n", ctypes.c_int64),
                ("pos", P), ("seq", P), ("seq_base", P), ("cu_seqlens", P), ("start_pos", P),
                ("ctx_len", P), ("order", P), ("max_seqlen", ctypes.c_int64), ("pool_rows", ctypes.c_int64),
                ("dst_capacity", ctypes.c_int64), ("max_ctx", ctypes.c_int64)]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    d = tmp_path_factory.mktemp("devcheck")
    src, lib = d / "driver.cpp", d / "libdevcheck.so"
    src.write_text(DRIVER)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-shared", "-fPIC", "-I", CSRC, str(src),
                    "-o", str(lib)], check=True)
    so = ctypes.CDLL(str(lib))
    so.first_violation.argtypes = [ctypes.POINTER(Inputs), ctypes.POINTER(ctypes.c_int64)]
    so.first_violation.restype = ctypes.c_int32

    def run(call, n, dst_kind=0, max_seqlen=0, pool_rows=0, dst_capacity=0, max_ctx=0, **arrays):
        keep = {}
        kw = {}
        for name, arr in arrays.items():
            dt = np.int32 if name in ("seq", "order") else np.int64
            keep[name] = np.ascontiguousarray(arr, dtype=dt)
            kw[name] = keep[name].ctypes.data
        x = Inputs(call=call, dst_kind=dst_kind, n=n, max_seqlen=max_seqlen, pool_rows=pool_rows,
                   dst_capacity=dst_capacity, max_ctx=max_ctx, **kw)
        where = ctypes.c_int64()
        code = so.first_violation(ctypes.byref(x), ctypes.byref(where))
        return code, where.value

    return run


def test_rope_rules(checker):
    pos = [0, 5, 7, 524288, 2 ** 40]
    ring = dict(call=ROPE, n=5, dst_kind=RING, dst_capacity=3)
    assert checker(pos=pos, seq=[0, 1, 2, 2, 0], **ring) == (OK, -1)
    assert checker(pos=[0, 5, -1, 3, 3], seq=[0, 1, 2, 2, 0], **ring) == (POSITION, 2)
    assert checker(pos=pos, seq=[0, 1, 3, 2, 0], **ring) == (RING_SEQ, 2)
    assert checker(pos=pos, seq=[0, -1, 2, 2, 0], **ring) == (RING_SEQ, 1)
    pool = dict(call=ROPE, n=3, dst_kind=POOL, dst_capacity=100)
    assert checker(pos=[0, 9, 49], seq=[0, 1, 1], seq_base=[10, 50], **pool) == (OK, -1)
    assert checker(pos=[0, 9, 50], seq=[0, 1, 1], seq_base=[10, 50], **pool) == (DST_RANGE, 2)   # row 100
    assert checker(pos=[0, 9, 5], seq=[0, -2, 1], seq_base=[10, 50], **pool) == (DST_RANGE, 1)
    assert checker(pos=[3, 0, 5], seq=[0, 1, 1], seq_base=[-10, 50], **pool) == (DST_RANGE, 0)  # row -7
    stage = dict(call=ROPE, n=4, dst_kind=STAGING)
    assert checker(pos=[0, 1, 2, 3], dst_capacity=4, **stage) == (OK, -1)
    assert checker(pos=[0, 1, 2, 3], dst_capacity=3, **stage) == (DST_RANGE, 3)


def test_prefill_rules(checker):
    swa = dict(call=SWA_PREFILL, n=3, max_seqlen=8)
    assert checker(cu_seqlens=[0, 8, 8, 11], start_pos=[0, 5, 2 ** 33], **swa) == (OK, -1)
    assert checker(cu_seqlens=[-1, 8, 8, 11], start_pos=[0, 5, 7], **swa) == (CU_SEQLENS, 0)
    assert checker(cu_seqlens=[0, 8, 7, 11], start_pos=[0, 5, 7], **swa) == (CU_SEQLENS, 1)   # decreasing
    assert checker(cu_seqlens=[0, 8, 8, 17], start_pos=[0, 5, 7], **swa) == (CU_SEQLENS, 2)   # 9 > 8
    assert checker(cu_seqlens=[0, 8, 8, 11], start_pos=[0, -5, 7], **swa) == (POSITION, 1)
    full = dict(call=FULL_PREFILL, n=2, max_seqlen=8, pool_rows=100)
    assert checker(cu_seqlens=[0, 8, 12], start_pos=[20, 30], seq_base=[0, 66], **full) == (OK, -1)  # 66+30+4 = 100
    assert checker(cu_seqlens=[0, 8, 12], start_pos=[20, 31], seq_base=[0, 66], **full) == (POOL_RANGE, 1)
    assert checker(cu_seqlens=[0, 8, 12], start_pos=[20, 30], seq_base=[-1, 66], **full) == (POOL_RANGE, 0)
    assert checker(cu_seqlens=[0, 8, 12], start_pos=[-20, 30], seq_base=[0, 66], **full) == (POSITION, 0)


def test_decode_rules(checker):
    assert checker(call=SWA_DECODE, n=3, pos=[0, 127, 2 ** 35]) == (OK, -1)
    assert checker(call=SWA_DECODE, n=3, pos=[0, -127, 5]) == (POSITION, 1)
    fd = dict(call=FULL_DECODE, n=3, max_ctx=50, pool_rows=100)
    assert checker(ctx_len=[1, 50, 20], seq_base=[0, 1, 80], **fd) == (OK, -1)
    assert checker(ctx_len=[1, 0, 20], seq_base=[0, 1, 80], **fd) == (CTX_LEN, 1)
    assert checker(ctx_len=[1, 51, 20], seq_base=[0, 1, 80], **fd) == (CTX_LEN, 1)
    assert checker(ctx_len=[1, 50, 21], seq_base=[0, 1, 80], **fd) == (POOL_RANGE, 2)
    assert checker(ctx_len=[1, 50, 20], seq_base=[0, -1, 80], **fd) == (POOL_RANGE, 1)


def test_vision_rules(checker):
    vit = dict(call=VIT, n=2, max_seqlen=4)
    assert checker(cu_seqlens=[0, 4, 8], order=[3, 2, 1, 0, 0, 2, 1, 3], **vit) == (OK, -1)
    assert checker(cu_seqlens=[0, 4, 8], **vit) == (OK, -1)                       # no order: row order
    assert checker(cu_seqlens=[0, 4, 8], order=[3, 2, 1, 0, 0, 4, 1, 3], **vit) == (ORDER, 1)
    assert checker(cu_seqlens=[0, 4, 8], order=[3, -1, 1, 0, 0, 2, 1, 3], **vit) == (ORDER, 0)
    assert checker(cu_seqlens=[0, 5, 8], order=[0] * 8, **vit) == (CU_SEQLENS, 0)


def test_release_library_reports_unchecked():
    """libhsw.so checks nothing and says so without touching a GPU."""
    hsw = pytest.importorskip("hybrid_sliding_window_amd.hsw")
    if hsw.hsw_device_checks_enabled():
        pytest.skip("HSW_CHECK_DEVICE=1 selects the checked build")
    assert hsw.hsw_device_check_status() == (0, -1, -1)
    chk = hsw.load_library(hsw.CHECKED_LIB_PATH)
    assert chk.hsw_device_checks_enabled() and chk.hsw_version().endswith("checked")
    for name in hsw.EXPORTED:
        assert hasattr(chk.lib, name)
