"""Checks of the attention kernels' gfx950 assembly for hazards the compiler cannot see.

The P·V products are inline assembly (their accumulators pinned to AGPRs) and the LDS reads
and waits are inline assembly too, so the compiler's hazard recognizer does not cover every
access around them. This module compiles the kernel source to device assembly with the
library's flags and checks three rules over every kernel instance:

* ``valu_mfma``: no MFMA reads a VGPR as its A or B operand within 2 wait states of a vector
  instruction that wrote it (an instruction counts 1 wait state, ``s_nop N`` N + 1).
* ``lds_pending``: no instruction reads or writes a VGPR while an LDS read into it is still
  outstanding by the ``lgkmcnt`` rule (LDS operations of a wave complete in order; scalar
  memory reads count in the same counter and are modelled as entries without registers).
* ``carried_mfma_write``: no register that an assembly statement lists in a ``; carry`` or
  ``; hold`` comment (operands the statement claims to rewrite but does not touch) was last
  written by an MFMA: the compiler would take the statement for the writer and drop the
  MFMA's wait states before the next reader.

The checks read straight-line instruction streams in program order (a label or a branch does
not reset the state), which is what the kernels' bodies are.

    python -m gqa_causal_prefill_amd.isa_check             # compile the source, check, report
    python -m gqa_causal_prefill_amd.isa_check --asm FILE  # check an existing assembly file
"""

from __future__ import annotations

import argparse
import os
import re
import subprocess
import sys
import tempfile
from dataclasses import dataclass, field

from . import build

SOURCE = os.path.join(build.PKG, "csrc", "gqa_prefill.hip")


@dataclass
class Inst:
    op: str
    operands: list
    carried: list = field(default_factory=list)   # registers named in a carry/hold comment


@dataclass
class Report:
    kernel: str
    instructions: int = 0
    mfmas: int = 0
    carried: int = 0
    violations: dict = field(default_factory=lambda: {"valu_mfma": [], "lds_pending": [], "carried_mfma_write": []})

    def ok(self) -> bool:
        return not any(self.violations.values())


_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"^-?\|?([va])(\d+)\|?$")


def registers(token: str) -> set:
    """VGPRs (``v``) and AGPRs (``a``) an operand names, as (file, index) pairs."""
    t = token.strip().rstrip(",")
    m = _RANGE.match(t)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(t)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def parse(text: str) -> dict:
    """Kernel name -> instruction stream, from compiler-written assembly."""
    kernels, cur = {}, None
    for line in text.split("\n"):
        m = re.match(r"^(_Z\S*_kernel\S*):", line)
        if m:
            cur = m.group(1)
            kernels[cur] = []
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        code, _, comment = line.partition(";")
        code = code.strip()
        carried = []
        m = re.search(r"\b(?:carry|hold)\b(.*)$", comment)
        if m:
            carried = m.group(1).split()
        if not code:
            if carried:
                kernels[cur].append(Inst("asm_hold", [], carried))
            continue
        if code.startswith(".") or code.endswith(":"):
            continue
        op, _, rest = code.partition(" ")
        operands = [o.strip() for o in rest.split(",")] if rest.strip() else []
        kernels[cur].append(Inst(op, operands, carried))
    return kernels


def _is_mfma(op: str) -> bool:
    return op.startswith("v_mfma") or op.startswith("v_smfmac")


def _is_valu(op: str) -> bool:
    return op.startswith("v_") and not _is_mfma(op)


def check(name: str, insts: list) -> Report:
    rep = Report(name, instructions=len(insts), mfmas=sum(1 for i in insts if _is_mfma(i.op)))
    # valu_mfma
    for k, ins in enumerate(insts):
        if not _is_mfma(ins.op) or len(ins.operands) < 3:
            continue
        srcs = registers(ins.operands[1]) | registers(ins.operands[2])
        ws, j = 0, k - 1
        while j >= 0 and ws < 2:
            prev = insts[j]
            if prev.op == "s_nop":
                ws += int(prev.operands[0], 0) + 1
            else:
                if _is_valu(prev.op) and prev.operands and registers(prev.operands[0]) & srcs:
                    rep.violations["valu_mfma"].append((j, k, prev.op, ins.op))
                ws += 1
            j -= 1
    # lds_pending
    queue = []
    for k, ins in enumerate(insts):
        if ins.op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", " ".join(ins.operands))
            if m:
                n = int(m.group(1))
                while len(queue) > n:
                    queue.pop(0)
            continue
        pending = set().union(*queue) if queue else set()
        if pending and (ins.op.startswith(("v_", "ds_", "buffer_", "global_"))):
            touched = set()
            for o in ins.operands:
                touched |= registers(o)
            if touched & pending:
                rep.violations["lds_pending"].append((k, ins.op))
        if ins.op.startswith(("ds_read", "ds_load")):
            queue.append(registers(ins.operands[0]))
        elif ins.op.startswith(("ds_", "s_load", "s_buffer_load")):
            queue.append(set())
    # carried_mfma_write
    last = {}
    for k, ins in enumerate(insts):
        for c in ins.carried:
            for r in registers(c):
                rep.carried += 1
                if r in last and _is_mfma(last[r][1]):
                    rep.violations["carried_mfma_write"].append((last[r][0], k, c))
        if ins.operands and ins.op.startswith(("v_", "ds_", "buffer_", "global_")):
            for r in registers(ins.operands[0]):
                last[r] = (k, ins.op)
        for c in ins.carried:
            for r in registers(c):
                last[r] = (k, "asm")
    return rep


def compile_asm(source: str, out: str) -> None:
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [build.hipcc(), *flags, f"-I{build.INCLUDE}", "--cuda-device-only", "-S", "-o", out, source]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--asm", help="check this assembly file instead of compiling the source")
    ap.add_argument("--source", default=SOURCE)
    a = ap.parse_args(argv)
    if a.asm:
        text = open(a.asm).read()
    else:
        with tempfile.TemporaryDirectory() as d:
            path = os.path.join(d, "kernels.s")
            compile_asm(a.source, path)
            text = open(path).read()
    bad = 0
    for name, insts in parse(text).items():
        rep = check(name, insts)
        v = rep.violations
        print(f"{name}: {rep.instructions} instructions, {rep.mfmas} MFMAs, {rep.carried} carried registers; "
              f"valu_mfma {len(v['valu_mfma'])}, lds_pending {len(v['lds_pending'])}, "
              f"carried_mfma_write {len(v['carried_mfma_write'])}")
        bad += not rep.ok()
    print("ok" if bad == 0 else f"{bad} kernel(s) with violations")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
