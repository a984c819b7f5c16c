"""Static check of a gfx950 wait-state rule for the encoder's inline-assembly
stores, in the assembly of the current sources.

A vector-memory instruction that reads an SGPR written by a VALU instruction
(v_readfirstlane / v_readlane, a compare or carry-out written to an SGPR
pair or VCC, ...) needs five wait states between the two; the compiler
inserts them for the instructions it generates, but does not look inside
inline assembly. The encoder's renormalisation store (`buffer_store_short
... idxen` inside an asm block, exec narrowed by `s_and_saveexec_b64` just
before it) carries no `s_nop`: its scalar operands, the slot descriptor and
the word offset, come from scalar instructions. This module proves that for
the compiled code: within the five wait states before every such store no
VALU instruction may write one of the store's SGPRs, and no label falls in
that window (a label would bring in paths not seen in the listing).
"""
from __future__ import annotations

import re

_STORE = re.compile(r"buffer_store_short (v\d+), (v\d+), (s\[\d+:\d+\]), (s\d+|\d+) idxen")
_LABEL = re.compile(r"^\.?\w+:")
WAIT_STATES = 5


def sgprs(tok: str) -> set:
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    if tok in ("vcc", "vcc_lo", "vcc_hi"):
        return {"vcc"}
    return set()


def valu_sgpr_writes(ins: str) -> set:
    """SGPRs a VALU instruction may write: any SGPR or VCC among its first two
    operands (destination, or the carry / compare result of VOP3 forms)."""
    parts = ins.split(None, 1)
    if not parts[0].startswith("v_") or len(parts) < 2:
        return set()
    out = set()
    for o in [p.strip() for p in parts[1].split(",")][:2]:
        out |= sgprs(o)
    return out


def check_lines(lines: list[str]) -> tuple[int, list[tuple[int, str]]]:
    """(stores checked, [(line, problem)]) for every idxen buffer store."""
    found, problems = 0, []
    for i, raw in enumerate(lines):
        t = raw.strip()
        m = _STORE.search(t)
        if not m:
            continue
        found += 1
        need = sgprs(m.group(3)) | sgprs(m.group(4))
        ws, j = 0, i - 1
        while ws < WAIT_STATES and j >= 0:
            u = lines[j].strip()
            j -= 1
            if not u or u.startswith(";"):
                continue
            if _LABEL.match(u):
                problems.append((i + 1, "label %s within %d wait states" % (u, WAIT_STATES)))
                break
            if u.startswith("s_nop"):
                ws += int(u.split()[1], 0) + 1
                continue
            hit = valu_sgpr_writes(u) & need
            if hit:
                problems.append((i + 1, "%s may write %s read by the store" % (u, sorted(hit, key=str))))
                break
            ws += 1
    return found, problems


def check_kernel(lines: list[str], symbol: str):
    s = next(i for i, l in enumerate(lines) if l.startswith(symbol + ":"))
    e = next(i for i in range(s, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return check_lines(lines[s + 1:e])


ENCODERS = ("_ZN2cg8k_encodeILb0EEEvNS_10EncodeArgsE", "_ZN2cg8k_encodeILb1EEEvNS_10EncodeArgsE")
