"""Static check of the matrix-core hazards in compiled gfx950 assembly.

The verify-attention kernel issues some MFMAs as inline asm, which the
compiler's hazard recognizer does not see.  This checker reads the assembly
(``hipcc --cuda-device-only -S``) and verifies, along every control-flow path
up to the needed distance, the two rules those instructions rely on
(CDNA3/CDNA4 ISA, MFMA dependency rules; a wait state is one instruction, or
N + 1 for ``s_nop N``):

* result: after an 8-pass MFMA, no instruction other than an MFMA that
  accumulates into exactly the same registers may read or write its result
  registers within RESULT_WAIT wait states;
* operand: no VALU instruction may write an MFMA's A, B or C operand registers
  within OPERAND_WAIT wait states before the MFMA.

Usage: python -m tree_verify_mla_amd.isa_check file.s [kernel-name-substring]
Exit status 1 and a listing of the violations if any rule is broken.
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass, field

RESULT_WAIT = 11   # 8-pass XDL write -> read/write by other instructions
OPERAND_WAIT = 2   # VALU write -> MFMA operand read

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")


def _regs(text: str) -> set:
    out = set()
    for kind, lo, hi, one in _REG.findall(text):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return out


@dataclass
class Inst:
    line: int
    op: str
    text: str
    defs: set = field(default_factory=set)
    uses: set = field(default_factory=set)
    waits: int = 1
    targets: tuple = ()
    falls: bool = True


def _parse_inst(lineno: int, text: str) -> Inst:
    body = text.split(";")[0].strip()
    op, _, rest = body.partition(" ")
    ins = Inst(lineno, op, body)
    operands = [o.strip() for o in _split_operands(rest)]
    if op == "s_nop":
        ins.waits = int(operands[0], 0) + 1 if operands and operands[0] else 1
    if op.startswith("s_cbranch"):
        ins.targets = (operands[0],)
    elif op == "s_branch":
        ins.targets = (operands[0],)
        ins.falls = False
    elif op in ("s_endpgm", "s_setpc_b64"):
        ins.falls = False
    # registers: stores and writes have no register result
    writes_first = not (op.startswith(("ds_write", "buffer_store", "global_store", "scratch_store",
                                       "flat_store", "s_")) or (op.startswith("buffer_load") and " lds" in body))
    if operands and writes_first and (op.startswith("v_") or op.startswith(("ds_", "buffer_", "global_", "scratch_", "flat_"))):
        ins.defs = _regs(operands[0])
        ins.uses = set().union(*[_regs(o) for o in operands[1:]]) if len(operands) > 1 else set()
    else:
        ins.uses = set().union(*[_regs(o) for o in operands]) if operands else set()
    return ins


def _split_operands(rest: str):
    depth, cur, out = 0, [], []
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            out.append("".join(cur))
            cur = []
        else:
            cur.append(ch)
    if "".join(cur).strip():
        out.append("".join(cur))
    return out


def parse_kernel(asm: str, name_sub: str):
    """Instructions and label positions of the first function whose symbol contains name_sub."""
    lines = asm.splitlines()
    start = None
    for i, l in enumerate(lines):
        if re.match(r"^[A-Za-z_.$][\w.$]*:", l) and name_sub in l and not l.startswith("."):
            start = i
            break
    if start is None:
        raise ValueError(f"kernel {name_sub!r} not found")
    insts, labels = [], {}
    for i in range(start + 1, len(lines)):
        l = lines[i]
        if l.startswith(".Lfunc_end"):
            break
        m = re.match(r"^(\.?L\w+|[A-Za-z_]\w*):", l)
        if m:
            labels[m.group(1)] = len(insts)
            continue
        s = l.strip()
        if not s or s.startswith((";", ".")):
            continue
        insts.append(_parse_inst(i + 1, s))
    return insts, labels


def _paths(insts, labels, i, budget, forward=True):
    """Yield (index, distance) of instructions reachable within `budget` wait states."""
    seen = {}
    stack = [(i, 0)]
    while stack:
        j, d = stack.pop()
        if forward:
            nxt = []
            ins = insts[j]
            if ins.falls and j + 1 < len(insts):
                nxt.append(j + 1)
            for t in ins.targets:
                if t in labels:
                    nxt.append(labels[t])
            for k in nxt:
                dk = d + insts[j].waits if j != i else d
                if dk >= budget or seen.get(k, 1 << 30) <= dk:
                    continue
                seen[k] = dk
                yield k, dk
                stack.append((k, dk))
        else:
            k = j - 1
            if k < 0:
                continue
            dk = d + insts[k].waits
            # straight-line predecessors only (labels end the backward walk)
            if k + 1 in labels.values() and k + 1 != i:
                continue
            if dk > budget or seen.get(k, 1 << 30) <= dk:
                continue
            seen[k] = dk
            yield k, dk
            stack.append((k, dk))


def check(asm: str, name_sub: str):
    insts, labels = parse_kernel(asm, name_sub)
    problems = []
    for i, ins in enumerate(insts):
        if not ins.op.startswith("v_mfma"):
            continue
        res = ins.defs
        for k, d in _paths(insts, labels, i, RESULT_WAIT):
            other = insts[k]
            touches = (other.defs | other.uses) & res
            if not touches:
                continue
            same_acc = other.op.startswith("v_mfma") and other.defs == res
            if not same_acc:
                problems.append(f"line {other.line}: {other.text!r} touches the result of the MFMA at "
                                f"line {ins.line} after {d} wait states (< {RESULT_WAIT})")
        operands = ins.uses
        for k, d in _paths(insts, labels, i, OPERAND_WAIT, forward=False):
            other = insts[k]
            if other.op.startswith("v_") and not other.op.startswith("v_mfma") and other.defs & operands:
                problems.append(f"line {other.line}: {other.text!r} writes an operand of the MFMA at "
                                f"line {ins.line} {d} wait states before it (< {OPERAND_WAIT})")
    return problems, sum(1 for x in insts if x.op.startswith("v_mfma"))


def main(argv):
    if len(argv) < 2:
        print(__doc__)
        return 2
    asm = open(argv[1]).read()
    name = argv[2] if len(argv) > 2 else "attn_bf16_kernel"
    problems, n = check(asm, name)
    for p in problems:
        print(p)
    print(f"{n} MFMAs checked, {len(problems)} hazard(s)")
    return 1 if problems else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
