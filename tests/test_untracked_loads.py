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
@pytest.mark.parametrize("src,kernel,n", [("swa_prefill.hip", "swa_prefill_kernel", 5),
                                          ("full_prefill.hip", "full_prefill_kernel", 9)])
def test_prefill_q_loads_are_never_touched_in_flight(src, kernel, n):
    asm = avc.compile_to_asm(os.path.join(CSRC, src))
    kernels = {k: v for k, v in avc.kernel_functions(asm).items() if kernel in k}
    assert len(kernels) == n
    for name, body in kernels.items():
        assert avc.check(body) == [], name


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_full_prefill_g16_kernel_keeps_its_loop_registers():
    """The G = 16 full-attention kernel (common and general bodies, with and
    without the fused q-RoPE) touches no register an untracked load may still
    be writing, and its common loop neither spills nor waits for every load
    in flight (a spill reload there is followed by vmcnt(0), which would also
    wait for the chunk loads the pipeline keeps in flight)."""
    asm = avc.compile_to_asm(os.path.join(CSRC, "full_prefill.hip"))
    kernels = {k: v for k, v in avc.kernel_functions(asm).items() if "full_prefill_pp_kernel" in k}
    assert len(kernels) == 2
    for name, body in kernels.items():
        assert avc.check(body) == [], name
        loops = loop_bodies(body)
        common = [b for b in loops.values() if not any("v_cvt_f32_f16" in l for l in b)]
        assert len(common) == 2, f"{name}: expected one common chunk loop per half"
        for b in common:
            assert not any("scratch_" in l for l in b), f"{name}: the common loop spills"
            assert not any("vmcnt(0)" in l for l in b), f"{name}: the common loop waits for every load"


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_windowed_sweep_kernels_keep_their_loop_registers():
    """The windowed sweep kernels (8 and 16 query heads per KV head, with
    and without the fused q-RoPE) touch no register an untracked load may
    still be writing, never spill, and wait for every load in flight only
    at the start of each of the two blocks of their loop (a spill reload
    would add a full wait, which also waits for the next q and chunks)."""
    asm = avc.compile_to_asm(os.path.join(CSRC, "swa_prefill.hip"))
    kernels = {k: v for k, v in avc.kernel_functions(asm).items() if "swa_sweep_kernel" in k}
    assert len(kernels) == 4
    for name, body in kernels.items():
        assert avc.check(body) == [], name
        assert not any("scratch_" in l for l in body), f"{name}: spills"
        loops = loop_bodies(body)
        main = [l.strip() for l in max(loops.values(), key=len)]
        code = [l for l in main if l and not l.startswith(";")]
        # (the compiler's own wait for the q loads sits next to the explicit
        # one: consecutive full waits are one wait point)
        points = sum("vmcnt(0)" in l and (i == 0 or "vmcnt(0)" not in code[i - 1]) for i, l in enumerate(code))
        assert points == 2, f"{name}: a full wait inside a block"


def loop_bodies(body):
    """Outermost loops of a function's assembly, by the compiler's block
    annotations ("Loop Header: Depth=1", "in Loop: Header=BBn_m"): header
    label -> the lines of the blocks in that loop.  (The P split of the
    general body converts fp16 to fp32 with v_cvt_f32_f16; the common body
    never does.)"""
    import re
    out, cur = {}, None
    for line in body:
        m = re.match(r"^\.?(LBB\w+|; %bb\.\d+):?", line)
        if m or line.startswith("; %bb."):
            h = re.search(r"Header=(BB\w+)", line)
            if "Loop Header: Depth=1" in line:
                cur = line.split(":")[0].lstrip(".").lstrip("L")
            else:
                cur = h.group(1) if h else None
            continue
        if cur is not None:
            out.setdefault(cur, []).append(line)
    return out
