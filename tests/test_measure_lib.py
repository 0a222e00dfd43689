"""The measurement-only library (libhsw_measure.so: a plain read of
item-shaped blocks that bench.py times beside the windowed decode) loads,
exports its entry point and refuses bad arguments on the host, launching
nothing (no GPU needed: every call here fails its argument checks)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "hybrid_sliding_window_amd", "libhsw_measure.so")
FAKE = 0x10000  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libhsw_measure.so not built (python -m hybrid_sliding_window_amd.build)")
    lib = ctypes.CDLL(LIB)
    f = lib.hsw_measure_read_items
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return lib


def test_exports_the_read_entry_point(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    assert " T hsw_measure_read_items" in out


@pytest.mark.parametrize("args", [
    (0, FAKE, FAKE, 4, 49152, 32768, 3072, FAKE),          # null K
    (FAKE, FAKE, FAKE, 4, 49152, 32768, 3072, 0),          # null sink
    (FAKE, FAKE, FAKE, 0, 49152, 32768, 3072, FAKE),       # no items
    (FAKE, FAKE, FAKE, 4, 49150, 32768, 3072, FAKE),       # K block not a multiple of 16 bytes
    (FAKE, FAKE, FAKE, 4, 49152, -16, 3072, FAKE),         # negative V block
    (FAKE + 8, FAKE, FAKE, 4, 49152, 32768, 3072, FAKE),   # misaligned K
])
def test_bad_arguments_are_refused_before_any_launch(lib, args):
    assert lib.hsw_measure_read_items(*args, None) == 1
