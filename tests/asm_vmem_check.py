"""Static check of untracked vector-memory loads in the gfx950 assembly of a
persistent kernel.  Test infrastructure only.

The windowed decode kernel issues the next item's loads as inline asm that
the compiler does not track, so they stay in flight while the current item
is computed, and waits for them with explicit `s_waitcnt vmcnt(N)`.  That is
correct only if no instruction reads or writes a VGPR while an untracked load
into it may still be in flight: a register copy or reuse that the register
allocator inserts between such a load and its wait sees stale data, or is
overwritten when the load lands (the kernel then computes garbage or faults).
The compiler cannot see this invariant, so this module checks it on the
assembly it produced.

Model: the untracked loads are the `global_load_*` instructions between
the `;;#ASMSTART` / `;;#ASMEND` markers that surround inline asm (those with
a VGPR destination fill registers, those into LDS only occupy a count).
Vector-memory operations complete in issue order, so `s_waitcnt vmcnt(N)`
retires every untracked load except the youngest N of them (ignoring the
tracked operations only retires fewer, which is the safe side).  The
kernel's main loop (the one issuing the most untracked loads) is scanned
block by block in execution order, header first and rotated latch blocks
last, twice, so the loads issued late in one iteration are followed into the
next.
"""
from __future__ import annotations

import os
import re
import subprocess

VREG = re.compile(r"(?<![\w\[])v\[(\d+):(\d+)\]|(?<![\w\[])v(\d+)\b")
WAIT_VM = re.compile(r"\bvmcnt\((\d+)\)")


def vregs(text: str) -> set:
    out = set()
    for m in VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def kernel_functions(asm: str) -> dict:
    """Kernel symbol -> its lines (from its label to .Lfunc_end)."""
    lines = asm.splitlines()
    out, i = {}, 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m:
            j = i + 1
            while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
                j += 1
            out[m.group(1)] = lines[i + 1:j]
            i = j
        i += 1
    return out


def _blocks(body):
    """[(label, loop header annotation, [(instruction, untracked?)])]."""
    blocks = [[None, "", []]]
    in_asm = False
    for raw in body:
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^\.(LBB\d+_\d+):(.*)$", s)
        if m:
            blocks.append([m.group(1), m.group(2), []])
            continue
        s = s.split(";")[0].strip()
        if s and not s.startswith("."):
            blocks[-1][2].append((s, in_asm))
    return blocks


def _untracked_load(ins, in_asm):
    op = ins.split()[0]
    return in_asm and op.startswith("global_load_dword") and "lds" not in op


def check(body):
    """List of (instruction, registers) touching an in-flight untracked load's
    destination inside the main loop; [] when the invariant holds."""
    blocks = _blocks(body)
    # main loop: the header whose loop issues the most untracked loads
    count = {}
    for lab, note, ins in blocks:
        m = re.search(r"Header=(BB\d+_\d+)", note)
        hdr = m.group(1) if m else (lab[1:] if lab and "Loop Header" in note else None)
        if hdr:
            count[hdr] = count.get(hdr, 0) + sum(_untracked_load(i, a) for i, a in ins)
    if not count or max(count.values()) == 0:
        return []
    hdr = max(count, key=count.get)
    loop = [b for b in blocks if b[0] == "L" + hdr or ("Header=" + hdr) in b[1]]
    h = next(k for k, b in enumerate(loop) if b[0] == "L" + hdr)
    order = loop[h:] + loop[:h]

    inflight = []   # ordered oldest -> youngest: sets of registers
    bad = {}
    for _ in range(2):
        for _, _, ins in order:
            for text, in_asm in ins:
                op = text.split()[0]
                if op == "s_waitcnt":
                    m = WAIT_VM.search(text)
                    if m:
                        n = int(m.group(1))
                        inflight = inflight[len(inflight) - n:] if n < len(inflight) else inflight
                        if n == 0:
                            inflight = []
                    continue
                live = set().union(*inflight) if inflight else set()
                operands = text[len(op):]
                if in_asm and op.startswith("global_load_lds"):
                    inflight.append(set())  # occupies a vmcnt slot, no VGPR destination
                    hit = vregs(operands) & live
                    if hit:
                        bad[text] = sorted(hit)
                    continue
                if _untracked_load(text, in_asm):
                    parts = [p.strip() for p in operands.split(",")]
                    hit = set().union(*[vregs(p) for p in parts[1:]]) & live
                    if hit:
                        bad[text] = sorted(hit)
                    inflight.append(vregs(parts[0]))
                    continue
                if op.startswith(("v_", "ds_", "global_", "buffer_", "scratch_", "flat_")):
                    hit = vregs(operands) & live
                    if hit:
                        bad[text] = sorted(hit)
    return sorted(bad.items())


def compile_to_asm(src: str) -> str:
    """Device assembly of one .hip source, built with the library's flags."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    from hybrid_sliding_window_amd import build as b
    flags = list(b.CFLAGS) + (b.RELAXED_NAN_FLAGS if os.path.basename(src) in b.RELAXED_NAN else [])
    cmd = [b.HIPCC, *flags, "--offload-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-2000:])
    return r.stdout
