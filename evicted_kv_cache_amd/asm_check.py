"""Check gfx950 device assembly for inline asm that follows a transcendental
VALU instruction too closely.

On CDNA3/CDNA4 a transcendental instruction (v_exp, v_log, v_rcp, v_rsq,
v_sqrt, v_sin, v_cos) needs one wait state before a following VALU
instruction reads its result, overwrites its result or overwrites one of
its sources.  The compiler inserts those wait states (an s_nop or an
independent instruction) for code it emits itself, but it does not look
inside inline asm, so an asm statement scheduled right after such an
instruction can read a stale register or corrupt the transcendental's
input.  This happened once in the fused decode: an inline v_fma_mix_f32
overwrote the register a v_exp_f32 was still reading, and the softmax
weight came out wrong for some lanes.

The build compiles each source that holds inline asm to device assembly and
runs `scan` over it; any hit fails the build.
"""
from __future__ import annotations

import re
from typing import List, Tuple

_TRANS = re.compile(r"^\s*(v_(?:exp|log|rcp|rsq|sqrt|sin|cos)_\w+)\s+(.*)$")
_FUNC = re.compile(r"^(_Z\S*|[A-Za-z_]\w*):")


def _vregs(operands: str) -> List[int]:
    """VGPR numbers named in an operand list (v7, v[4:7]); other operands ignored."""
    out: List[int] = []
    for tok in operands.split(","):
        tok = tok.strip()
        if not tok:
            continue
        tok = tok.split()[0]
        m = re.fullmatch(r"v(\d+)", tok)
        if m:
            out.append(int(m.group(1)))
            continue
        m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
        if m:
            out.extend(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _split_operands(line: str) -> Tuple[List[int], List[int]]:
    """(destination VGPRs, source VGPRs) of one VALU line: the first operand
    is the destination."""
    parts = line.strip().split(None, 1)
    if len(parts) < 2:
        return [], []
    ops = [o.strip() for o in parts[1].split(",")]
    return _vregs(ops[0]), _vregs(",".join(ops[1:]))


def scan(asm_text: str) -> List[str]:
    """Return one message per transcendental instruction whose very next
    instruction comes from inline asm and touches its registers."""
    lines = asm_text.split("\n")
    hits: List[str] = []
    func = "?"
    for i, line in enumerate(lines):
        fm = _FUNC.match(line)
        if fm:
            func = fm.group(1)
        if not _TRANS.match(line):
            continue
        t_dst, t_src = _split_operands(line)
        j, in_asm = i + 1, False
        while j < len(lines):
            s = lines[j].strip()
            if s.startswith(";;#ASMSTART"):
                in_asm = True
            elif s.startswith(";;#ASMEND"):
                in_asm = False
            elif s and not s.startswith(";") and not s.endswith(":") and not s.startswith("."):
                break
            j += 1
        if j >= len(lines) or not in_asm:
            continue
        a_dst, a_src = _split_operands(lines[j])
        if set(t_dst) & set(a_src) or set(t_src) & set(a_dst) or set(t_dst) & set(a_dst):
            hits.append(f"{func}: line {i + 1}: '{line.strip()}' followed by inline asm '{lines[j].strip()}'")
    return hits
