"""Static check of untracked vector-memory loads in the gfx950 assembly of
the attention kernels.  Test infrastructure only.

Several kernels issue loads as inline asm that the compiler does not track:
the windowed decode kernel's next-item K/q loads (in flight while the
current item is computed), and the prefill kernels' q loads (in flight while
the first chunk loads are issued, then covered by the pipeline's first
explicit wait).  Completion is awaited with explicit `s_waitcnt vmcnt(N)`.
That is correct only if no instruction reads or writes a VGPR while an
untracked load into it may still be in flight: a register copy or reuse that
the register allocator inserts between such a load and its wait sees stale
data, or is overwritten when the load lands (the kernel then computes
garbage or faults).  The compiler cannot see this invariant, so this module
checks it on the assembly it produced.

Model: the untracked loads are the `global_load_*` instructions between
the `;;#ASMSTART` / `;;#ASMEND` markers that surround inline asm (those with
a VGPR destination fill registers, those into LDS only occupy a count).
Vector-memory operations complete in issue order, so `s_waitcnt vmcnt(N)`
retires every untracked load except the youngest N of them (ignoring the
tracked operations only retires fewer, which is the safe side).  The state
at a point is the queue of untracked loads that may be in flight there,
youngest last; the analysis runs over the kernel's control-flow graph (basic
blocks split at labels, fall-through markers and branches), joins the queues
of a block's predecessors entry by entry from the youngest (a register may
be in flight if it is on any path), and iterates to a fixed point, so loops
carry the loads issued late in one iteration into the next.  The compiler
lowers `if (c) {A} else {B}` with a flag: one branch sets an SGPR pair to -1
or 0 (`s_mov_b64`) and a later block branches on `s_andn2_b64 vcc, exec,
pair`; to keep such paths apart, the state also carries the SGPR pairs known
to hold 0 or -1 (and vcc when derived from them), branches whose outcome
that fixes follow one edge only, and queues are joined only between states
with the same known values.
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
    """Basic blocks: [(label or None, [(instruction, untracked?)])], split at
    labels, `; %bb.N:` fall-through markers and after every branch."""
    blocks = [[None, []]]
    in_asm = False
    for raw in body:
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^\.(LBB\d+_\d+):", s)
        if m or re.match(r"^; %bb\.\d+:", s):
            blocks.append([m.group(1) if m else None, []])
            continue
        s = s.split(";")[0].strip()
        if s and not s.startswith("."):
            blocks[-1][1].append((s, in_asm))
            op = s.split()[0]
            if op.startswith("s_cbranch") or op == "s_branch":
                blocks.append([None, []])
    return blocks


def _successors(blocks):
    labels = {lab: i for i, (lab, _) in enumerate(blocks) if lab}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        out = []
        last = ins[-1][0].split() if ins else [""]
        if last[0].startswith("s_cbranch") or last[0] == "s_branch":
            tgt = last[-1].lstrip(".")
            if tgt in labels:
                out.append(labels[tgt])
        if last[0] not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    return succ


def _untracked_load(ins, in_asm):
    op = ins.split()[0]
    return in_asm and op.startswith("global_load_dword") and "lds" not in op


def _join(a, b):
    n = max(len(a), len(b))
    a = [set()] * (n - len(a)) + list(a)
    b = [set()] * (n - len(b)) + list(b)
    return [x | y for x, y in zip(a, b)]


def _step(state, text, in_asm, bad=None):
    """Apply one instruction to the in-flight queue; record touches in bad."""
    op = text.split()[0]
    if op == "s_waitcnt":
        m = WAIT_VM.search(text)
        if m:
            n = int(m.group(1))
            state = state[len(state) - n:] if 0 < n < len(state) else (state if n else [])
        return state
    live = set().union(*state) if state else set()
    operands = text[len(op):]
    if in_asm and op.startswith("global_load_lds"):
        hit = vregs(operands) & live
        state = (state + [set()])[-64:]  # occupies a vmcnt slot, no VGPR destination
    elif _untracked_load(text, in_asm):
        parts = [p.strip() for p in operands.split(",")]
        hit = set().union(*[vregs(p) for p in parts[1:]]) & live
        state = (state + [vregs(parts[0])])[-64:]
    elif op.startswith(("v_", "ds_", "global_", "buffer_", "scratch_", "flat_")):
        hit = vregs(operands) & live
    else:
        hit = set()
    if hit and bad is not None:
        bad[text] = sorted(set(bad.get(text, [])) | hit)
    return state


SREG = re.compile(r"^(?:s\[(\d+):(\d+)\]|s(\d+)|vcc)$")


def _sdst(text):
    """Scalar registers an instruction writes (first operand of SALU ops, the
    vcc / sdst of VOPC compares), as a set of 's<n>' / 'vcc' names."""
    op = text.split()[0]
    args = [p.strip() for p in text[len(op):].split(",")]
    first = args[0] if args and args[0] else ""
    if op.startswith("v_cmp"):
        return {"vcc"} if op.endswith("_e32") else _snames(first)
    if op.startswith("s_") and not op.startswith(("s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier",
                                                    "s_set", "s_endpgm", "s_cmp", "s_bitcmp", "s_sleep")):
        return _snames(first)
    if op.startswith("s_cmp") or op.startswith("s_bitcmp"):
        return set()
    return set()


def _snames(tok):
    m = SREG.match(tok)
    if not m:
        return set()
    if tok == "vcc":
        return {"vcc"}
    if m.group(3) is not None:
        return {"s" + m.group(3)}
    return {"s%d" % r for r in range(int(m.group(1)), int(m.group(2)) + 1)}


def _consts_step(consts, text):
    """Track SGPR pairs holding 0 / -1 and vcc derived from them."""
    op = text.split()[0]
    args = [p.strip() for p in text[len(op):].split(",")]
    out = dict(consts)
    for k in list(out):
        names = _snames(k) if k != "vcc" else {"vcc"}
        if names & _sdst(text):
            del out[k]
    if op == "s_mov_b64" and len(args) == 2 and args[1] in ("-1", "0") and SREG.match(args[0]):
        out[args[0]] = int(args[1])
    elif op in ("s_andn2_b64", "s_and_b64") and len(args) == 3 and args[0] == "vcc" and args[1] == "exec" \
            and args[2] in consts:
        c = consts[args[2]]
        nonzero = (c == 0) if op == "s_andn2_b64" else (c == -1)
        out["vcc"] = 1 if nonzero else 0
    return out


def _successors_known(blocks, succ, i, consts):
    ins = blocks[i][1]
    if not ins:
        return succ[i]
    last = ins[-1][0].split()
    if last[0] in ("s_cbranch_vccnz", "s_cbranch_vccz") and "vcc" in consts and len(succ[i]) == 2:
        taken = (consts["vcc"] == 1) == (last[0] == "s_cbranch_vccnz")
        return [succ[i][0]] if taken else [succ[i][1]]
    return succ[i]


def check(body):
    """List of (instruction, registers) touching a register that an
    untracked load may still be writing; [] when the invariant holds."""
    blocks = _blocks(body)
    succ = _successors(blocks)
    state_in = {(0, frozenset()): []}   # (block, known SGPR values) -> queue
    work = [(0, frozenset())]
    while work:
        key = work.pop()
        i, known = key
        st, consts = state_in[key], dict(known)
        for text, in_asm in blocks[i][1]:
            st = _step(st, text, in_asm)
            consts = _consts_step(consts, text)
        for j in _successors_known(blocks, succ, i, consts):
            k2 = (j, frozenset(consts.items()))
            new = st if k2 not in state_in else _join(state_in[k2], st)
            if k2 not in state_in or new != state_in[k2]:
                state_in[k2] = new
                work.append(k2)
    bad = {}
    for (i, known), st in state_in.items():
        for text, in_asm in blocks[i][1]:
            st = _step(st, text, in_asm, bad)
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
