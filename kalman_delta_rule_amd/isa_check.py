"""Build-time check of the gfx950 device assembly of this library's kernels.

One matrix-core dependency is not covered by the compiler's wait-state
insertion: a matrix product whose accumulator input (SrcC) is the result of
a product of a *different* opcode issued shortly before.  The matrix pipe
forwards results between back-to-back products of the same opcode; across
opcodes (for example a 16x16x32 bf16 product feeding a 16x16x16 bf16 one)
the second product reads a stale accumulator unless enough independent
instructions separate them.  Measured on gfx950 with a hand-scheduled
sequence: four wait states give a wrong result, eight the right one.

The kernels avoid the pattern by keeping every accumulation chain on one
opcode.  This module scans the compiled assembly and reports any remaining
occurrence, so that a code change cannot bring it back silently:

    python -m kalman_delta_rule_amd.isa_check  (also run by build.py)

Wait states are counted along every path from the producing product (each
instruction counts one, ``s_nop N`` counts N + 1), following branches.

It also rejects any function call in these sources' device code
(``s_swappc_b64``): their kernels keep each role's work inlined, and an
outlined call spills the caller's live registers to scratch on every step.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from typing import Dict, List, Tuple

# wait states required between a product and a different-opcode product
# reading its result as the accumulator (8 measured sufficient; keep a margin)
MIN_WAIT_STATES = 10

_VREG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)\b")


def _regs(tok: str) -> set:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    return set()


def parse_kernels(asm_text: str) -> Dict[str, List[str]]:
    """Instruction lists (labels kept as 'name:' entries) per kernel symbol."""
    kernels: Dict[str, List[str]] = {}
    cur = None
    for raw in asm_text.splitlines():
        m = re.match(r"^(_Z\w+):", raw)
        if m:
            cur = m.group(1)
            kernels[cur] = []
            continue
        if cur is None:
            continue
        if raw.startswith(".Lfunc_end"):
            cur = None
            continue
        t = raw.split(";")[0].strip()
        if not t:
            continue
        if t.startswith(".") and not t.endswith(":"):
            continue
        kernels[cur].append(t)
    return kernels


def _operands(ins: str) -> List[str]:
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def find_hazards(instrs: List[str], min_ws: int = MIN_WAIT_STATES) -> List[Tuple[str, str, int]]:
    """(producer, consumer, wait states) for each different-opcode accumulator
    dependency closer than ``min_ws``."""
    labels = {t[:-1]: i for i, t in enumerate(instrs) if t.endswith(":")}
    out = []
    for i, ins in enumerate(instrs):
        if not ins.startswith("v_mfma"):
            continue
        opc = ins.split()[0]
        ops = _operands(ins)
        if not ops:
            continue
        dst = _regs(ops[0])
        stack = [(i + 1, 0)]
        seen = set()
        while stack:
            j, ws = stack.pop()
            while j < len(instrs) and ws < min_ws:
                if (j, ws) in seen:
                    break
                seen.add((j, ws))
                u = instrs[j]
                if u.endswith(":"):
                    j += 1
                    continue
                op = u.split()[0]
                if op == "s_nop":
                    ws += int(u.split()[1], 0) + 1
                    j += 1
                    continue
                uops = _operands(u)
                if op.startswith("v_mfma") and len(uops) >= 4:
                    if (_regs(uops[3]) & dst) and op != opc:
                        out.append((ins, u, ws))
                    if _regs(uops[0]) & dst:
                        break  # the producer's result is overwritten on this path
                elif op.startswith("v_") and uops and (_regs(uops[0]) & dst):
                    break      # overwritten by a VALU op
                ws += 1
                if op == "s_branch":
                    tgt = u.split()[1]
                    if tgt in labels:
                        j = labels[tgt]
                        continue
                    break
                if op.startswith("s_cbranch"):
                    tgt = u.split()[1]
                    if tgt in labels:
                        stack.append((labels[tgt], ws))
                if op == "s_endpgm" or op == "s_setpc_b64":
                    break
                j += 1
    return out


def find_calls(instrs: List[str]) -> List[str]:
    """Function calls (outlined device functions) in one body."""
    return [ins for ins in instrs if ins.startswith("s_swappc_b64") or ins.startswith("s_call_b64")]


def device_asm(src: str, include_dirs: List[str], hipcc: str, flags: List[str]) -> str:
    """gfx950 assembly of one source file (device side only)."""
    cmd = ([hipcc] + [f for f in flags if f not in ("-shared", "-fPIC")]
           + ["--cuda-device-only", "-S", "-o", "-"]
           + sum([["-I", d] for d in include_dirs], []) + [src])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed for %s:\n%s" % (src, res.stderr[-2000:]))
    return res.stdout


def check_sources(sources: List[str], include_dirs: List[str], hipcc: str,
                  flags: List[str], verbose: bool = False) -> List[str]:
    problems = []
    for src in sources:
        kernels = parse_kernels(device_asm(src, include_dirs, hipcc, flags))
        for name, instrs in kernels.items():
            for call in find_calls(instrs):
                problems.append("%s %s: device-side call '%s' (an outlined function)"
                                % (os.path.basename(src), name[:60], call))
            hz = find_hazards(instrs)
            if verbose:
                print("isa-check %s: %s (%d products): %d hazard(s)"
                      % (os.path.basename(src), name[:80],
                         sum(1 for x in instrs if x.startswith("v_mfma")), len(hz)), flush=True)
            for a, b, ws in hz:
                problems.append("%s %s: '%s' then '%s' after %d wait states"
                                % (os.path.basename(src), name[:60], a, b, ws))
    return problems


if __name__ == "__main__":
    from kalman_delta_rule_amd import build as kbuild
    probs = kbuild.run_isa_check(verbose=True)
    for p in probs:
        print(p)
    sys.exit(1 if probs else 0)
