"""Wait-state checks on the gfx950 assembly of the kernels.

The kernels issue their MFMAs through inline asm, so the compiler inserts no
wait states for them.  This module scans the generated assembly for the MFMA
hazards that software must cover on CDNA3/CDNA4 and reports every place where
too few wait states separate two dependent instructions.  The limits are
conservative (at least as large as the ISA's requirement for any MFMA shape the
kernels use):

  * VALU write of a register -> MFMA reads it (A, B or C operand): 4 wait states
    (the ISA asks for 2);
  * MFMA write -> any other instruction reads or writes that register: 18
    (the ISA asks for up to 18, for 16-pass MFMAs);
  * MFMA write -> MFMA reads it as A or B, or as a C operand that is not the
    identical register range: 18;
  * MFMA reads a register as its C operand -> a non-MFMA instruction writes it: 18;
  * transcendental VALU op (v_exp, v_log, v_rcp, v_rsq, v_sqrt, v_sin, v_cos)
    writes a register -> a non-transcendental VALU op reads it: 1 (as the ISA asks;
    the compiler itself inserts exactly this many).

`check_untracked_loads` covers the vector memory loads issued through inline
asm (the compiler does not count them in the vmcnt waits it inserts): from such
a load until an `s_waitcnt vmcnt(N)` with at least N vector memory operations
issued after it, no instruction may read or write its destination registers.

Every instruction provides one wait state and `s_nop N` provides N + 1.  Control
flow is followed both ways: a label's predecessors are the fall-through and
every branch to it; a conditional branch continues to its target and falls
through.
"""
from __future__ import annotations

import dataclasses
import re

VALU_TO_MFMA = 4
MFMA_RESULT = 18
TRANS_RESULT = 1
_TRANS = ("v_exp_", "v_log_", "v_rcp_", "v_rsq_", "v_sqrt_", "v_sin_", "v_cos_")

_REG = re.compile(r"^([vas])(?:\[(\d+):(\d+)\]|(\d+))$")


@dataclasses.dataclass
class Insn:
    idx: int
    op: str
    operands: list
    text: str
    inline_asm: bool = False  # between the compiler's ASMSTART / ASMEND markers


def _regs(tok):
    tok = tok.strip()
    m = _REG.match(tok)
    if not m:
        return set()
    kind = m.group(1)
    if m.group(4) is not None:
        lo = hi = int(m.group(4))
    else:
        lo, hi = int(m.group(2)), int(m.group(3))
    return {(kind, r) for r in range(lo, hi + 1)}


def _split_operands(rest):
    rest = rest.split(";")[0].split("//")[0].strip()
    if not rest:
        return []
    return [t.strip() for t in rest.split(",")]


def parse_function(asm: str, name: str):
    """Instructions and labels of one function of an amdgcn .s file."""
    lines = asm.splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    insns, labels = [], {}
    in_asm = False
    for l in lines[start + 1:]:
        raw = l.strip()
        if raw.startswith(";;#ASMSTART"):
            in_asm = True
        elif raw.startswith(";;#ASMEND"):
            in_asm = False
        s = l.split(";")[0].split("//")[0].strip()
        if s.startswith(".Lfunc_end"):
            break
        if not s:
            continue
        if s.endswith(":") and not s.startswith("s_") and not s.startswith("v_"):
            labels[s[:-1]] = len(insns)
            continue
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        op = parts[0]
        ops = _split_operands(parts[1]) if len(parts) > 1 else []
        insns.append(Insn(len(insns), op, ops, s, in_asm))
    return insns, labels


def _wait_states(insn: Insn) -> int:
    if insn.op == "s_nop":
        return int(insn.operands[0], 0) + 1
    return 1


def _is_branch(insn):
    return insn.op.startswith("s_branch") or insn.op.startswith("s_cbranch")


def _ends_flow(insn):
    return insn.op in ("s_branch", "s_endpgm", "s_setpc_b64")


def _successors(insns, labels, i):
    insn = insns[i]
    out = []
    if _is_branch(insn):
        out.append(labels[insn.operands[0]])
    if not _ends_flow(insn) and i + 1 < len(insns):
        out.append(i + 1)
    return out


def _predecessors(insns, labels):
    preds = {i: [] for i in range(len(insns))}
    for i in range(len(insns)):
        for j in _successors(insns, labels, i):
            preds[j].append(i)
    return preds


def is_mfma(insn):
    return insn.op.startswith("v_mfma")


def _is_valu(insn):
    return insn.op.startswith("v_") and not is_mfma(insn)


def _valu_writes(insn):
    if not insn.operands:
        return set()
    w = _regs(insn.operands[0])
    if insn.op.startswith(("v_permlane", "v_swap")) and len(insn.operands) > 1:
        w |= _regs(insn.operands[1])
    return {r for r in w if r[0] in "va"}


def _all_regs(insn):
    out = set()
    for t in insn.operands:
        out |= _regs(t)
    return {r for r in out if r[0] in "va"}


def _mfma_parts(insn):
    dst = _regs(insn.operands[0])
    a = _regs(insn.operands[1])
    b = _regs(insn.operands[2])
    c = _regs(insn.operands[3]) if len(insn.operands) > 3 else set()
    return dst, a, b, c


def _walk(start_list, step, budget, visit):
    """Depth-first walk; `visit(i, used)` returns False to stop that path."""
    stack = [(i, 0) for i in start_list]
    seen = {}
    while stack:
        i, used = stack.pop()
        if used >= budget or seen.get(i, budget + 1) <= used:
            continue
        seen[i] = used
        if not visit(i, used):
            continue
        for j in step(i):
            stack.append((j, used + _WS[i]))


_WS = None


def check(insns, labels):
    """Return a list of human-readable hazard reports (empty when clean)."""
    global _WS
    _WS = [_wait_states(x) for x in insns]
    preds = _predecessors(insns, labels)
    succ = {i: _successors(insns, labels, i) for i in range(len(insns))}
    problems = []
    for m in (x for x in insns if is_mfma(x)):
        dst, a, b, c = _mfma_parts(m)
        srcs = a | b | c

        # VALU writes of an operand shortly before the MFMA
        def back(i, used, m=m, srcs=srcs):
            x = insns[i]
            if _is_valu(x) and _valu_writes(x) & srcs:
                problems.append(f"VALU write -> MFMA operand with {used} wait states: '{x.text}' before '{m.text}'")
            return True
        _walk(preds[m.idx], lambda i: preds[i], VALU_TO_MFMA, back)

        # uses of the result, and writes of the C operand, shortly after the MFMA
        def fwd(i, used, m=m, dst=dst, c=c):
            x = insns[i]
            if is_mfma(x):
                d2, a2, b2, c2 = _mfma_parts(x)
                if (a2 | b2) & dst:
                    problems.append(f"MFMA result -> MFMA A/B after {used} wait states: '{m.text}' then '{x.text}'")
                if c2 & dst and c2 != dst:
                    problems.append(f"MFMA result -> overlapping MFMA C after {used} wait states: '{m.text}' then '{x.text}'")
                if d2 & dst and d2 != dst:
                    problems.append(f"MFMA result -> overlapping MFMA write after {used}: '{m.text}' then '{x.text}'")
                return not (d2 == dst and c2 == dst)  # an accumulate into the same range continues the chain
            if x.op in ("s_nop", "s_waitcnt") or x.op.startswith("s_") and not _all_regs(x):
                return True
            regs = _all_regs(x)
            if regs & dst:
                problems.append(f"MFMA result -> '{x.op}' after {used} wait states: '{m.text}' then '{x.text}'")
            if _is_valu(x) and _valu_writes(x) & c and c != dst:
                problems.append(f"MFMA C read -> VALU write after {used} wait states: '{m.text}' then '{x.text}'")
            return True
        _walk(succ[m.idx], lambda i: succ[i], MFMA_RESULT, fwd)

    for tr in (x for x in insns if x.op.startswith(_TRANS)):
        written = _valu_writes(tr)

        def tfwd(i, used, tr=tr, written=written):
            x = insns[i]
            if _is_valu(x) and not x.op.startswith(_TRANS) and set().union(*[_regs(o) for o in x.operands[1:]] or [set()]) & written:
                problems.append(f"trans result -> VALU read after {used} wait states: '{tr.text}' then '{x.text}'")
            return True
        _walk(succ[tr.idx], lambda i: succ[i], TRANS_RESULT, tfwd)
    return sorted(set(problems))


_VMEM = ("global_load", "global_store", "global_atomic", "buffer_load", "buffer_store", "buffer_atomic",
         "flat_load", "flat_store", "flat_atomic", "scratch_load", "scratch_store")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")


def _is_vmem(insn):
    return insn.op.startswith(_VMEM)


def check_untracked_loads(insns):
    """Reports for inline-asm vector loads whose registers are used before a covering wait.

    Straight-line code is required between such a load and its wait: a branch in
    between is reported as well.
    """
    problems = []
    for ld in insns:
        if not (ld.inline_asm and ld.op.startswith(("global_load", "buffer_load")) and "lds" not in ld.op):
            continue
        dst = {r for r in _regs(ld.operands[0]) if r[0] in "va"}
        newer = 0
        for x in insns[ld.idx + 1:]:
            if x.op == "s_waitcnt":
                m = _VMCNT.search(x.text)
                if m and newer >= int(m.group(1)):
                    break
                continue
            if _is_branch(x) or _ends_flow(x):
                problems.append(f"'{ld.text}': control flow '{x.text}' before its wait")
                break
            if _all_regs(x) & dst:
                problems.append(f"'{ld.text}': '{x.text}' uses its registers before its wait")
            if _is_vmem(x):
                newer += 1
        else:
            problems.append(f"'{ld.text}': never awaited")
    return problems
