"""The untracked loads of the attention kernels (the windowed decode
kernel's next-item loads, the prefill kernels' q loads): no instruction of
the compiled kernels touches a register such a load may still be writing
(checked on the gfx950 assembly the build flags produce; CPU only, hipcc
cross-compiles)."""
import os
import shutil

import pytest

import asm_vmem_check as avc

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "hybrid_sliding_window_amd", "csrc")

# A loop that issues two untracked loads per iteration and waits for the
# previous iteration's with vmcnt(2); the copy reads a register whose load
# is still in flight.
_BAD = """_Zfake:
.LBB0_1:                                ; =>This Inner Loop Header: Depth=1
	;;#ASMSTART
	global_load_dwordx4 v[10:13], v[2:3], off
	;;#ASMEND
	;;#ASMSTART
	global_load_dwordx4 v[14:17], v[4:5], off
	;;#ASMEND
	v_mov_b32_e32 v20, v14
	;;#ASMSTART
	s_waitcnt vmcnt(2)
	;;#ASMEND
	v_mfma_f32_16x16x32_bf16 v[24:27], v[10:13], v[14:17], 0
	s_cbranch_scc1 .LBB0_1
.Lfunc_end0:
"""


def test_checker_flags_a_read_of_an_inflight_register():
    body = avc.kernel_functions(_BAD)["_Zfake"]
    bad = dict(avc.check(body))
    assert "v_mov_b32_e32 v20, v14" in bad
    # vmcnt(2) retires the previous iteration's loads but leaves this
    # iteration's two in flight, so the MFMA that reads them is flagged too
    assert any(k.startswith("v_mfma") for k in bad)


def test_checker_accepts_uses_after_the_covering_wait():
    good = _BAD.replace("\tv_mov_b32_e32 v20, v14\n", "").replace("vmcnt(2)", "vmcnt(0)")
    assert avc.check(avc.kernel_functions(good)["_Zfake"]) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_swa_decode_untracked_loads_are_never_touched_in_flight():
    asm = avc.compile_to_asm(os.path.join(CSRC, "swa_decode.hip"))
    kernels = {k: v for k, v in avc.kernel_functions(asm).items() if "swa_decode_kernel" in k}
    assert len(kernels) == 10  # per q/KV group size, with and without the fused q-RoPE
    for name, body in kernels.items():
        assert avc.check(body) == [], name


# An untracked q load before the loop, read by the loop's first MFMA before
# the wait that covers it (the loop's only wait retires older loads only).
_BAD_PROLOGUE = """_Zfake2:
	;;#ASMSTART
	global_load_dwordx4 v[30:33], v[2:3], off
	;;#ASMEND
	;;#ASMSTART
	s_mov_b32 m0, s4
	global_load_lds_dwordx4 v[4:5], off
	;;#ASMEND
.LBB1_1:                                ; =>This Inner Loop Header: Depth=1
	v_mfma_f32_16x16x32_bf16 v[24:27], v[10:13], v[30:33], 0
	;;#ASMSTART
	s_mov_b32 m0, s5
	global_load_lds_dwordx4 v[6:7], off
	;;#ASMEND
	s_waitcnt vmcnt(1)
	s_cbranch_scc1 .LBB1_1
.Lfunc_end1:
"""


def test_checker_follows_prologue_loads_into_the_loop():
    bad = dict(avc.check(avc.kernel_functions(_BAD_PROLOGUE)["_Zfake2"]))
    assert any(k.startswith("v_mfma") for k in bad)
    # waiting for all but the newest LDS load first covers q
    good = _BAD_PROLOGUE.replace(".LBB1_1:                                ; =>This Inner Loop Header: Depth=1\n",
                                 ".LBB1_1:                                ; =>This Inner Loop Header: Depth=1\n"
                                 "\ts_waitcnt vmcnt(1)\n")
    assert avc.check(avc.kernel_functions(good)["_Zfake2"]) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
@pytest.mark.parametrize("src,kernel,n", [("swa_prefill.hip", "swa_prefill_kernel", 9),
                                          ("full_prefill.hip", "full_prefill_kernel", 9)])
def test_prefill_q_loads_are_never_touched_in_flight(src, kernel, n):
    asm = avc.compile_to_asm(os.path.join(CSRC, src))
    kernels = {k: v for k, v in avc.kernel_functions(asm).items() if kernel in k}
    assert len(kernels) == n
    for name, body in kernels.items():
        assert avc.check(body) == [], name
