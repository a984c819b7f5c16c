"""Static check of the decoder's untracked prefetch loads in gfx950 assembly.

The decoder loads the next block of each chain's word stream with a
buffer_load_dword written as inline assembly (marked by the `s_nop 4` before
it), so the compiler does not wait for it; the code waits itself with
s_waitcnt vmcnt(k) sized by how many vector-memory operations were issued
since. The compiler still treats the destination register as written when
the instruction issues: it may copy it, or hand it to another value once the
prefetched word is dead, while the load is still in flight. This module
compiles the kernels to assembly with the library's own flags and proves, by
a data-flow pass over each decoder's basic blocks, that no instruction other
than the stream refill reads, copies or overwrites such a register before a
wait that covers the load on every path.

Model: a load is complete after `s_waitcnt vmcnt(k)` once at least k
vector-memory instructions were issued after it on the path (gfx9 retires
them in order). Paths are told apart by the constant 64-bit condition flags
the compiler's structurizer sets with `s_mov_b64 s[a:b], 0 / -1` and tests
with `s_and(n2)_b64 vcc, exec, s[a:b]` before a vccz/vccnz branch; other
branches are taken both ways. The refill itself (ds_write of the prefetched
word into the ring) is reported separately: its wait depends on the loop
age, which this model does not follow.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PAIR = r"s\[(\d+):(\d+)\]"
_VMEM = re.compile(r"(buffer_|global_|flat_|scratch_)\w+")
_WAIT = re.compile(r"s_waitcnt .*vmcnt\((\d+)\)")
_LOAD = re.compile(r"buffer_load_dword (v\d+),")
_MOV64 = re.compile(r"s_mov_b64 " + PAIR + r", (-1|0)$")
_ANDVCC = re.compile(r"s_(and|andn2)_b64 vcc, exec, " + PAIR + r"$")
_SWRITE = re.compile(r"s_\w+ " + PAIR)
_VCCW = re.compile(r"(v_cmp\w*|s_\w+) vcc|v_cmp\w*_e32")
_CAP = 11  # counts above the largest vmcnt the kernels wait for are equivalent


def compile_asm(out_path: str) -> None:
    from kv_cache_compression_encode_amd import build as B

    cmd = [B.HIPCC, *[f for f in B.COMMON if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "cg_kernels.hip"), "-o", out_path]
    subprocess.check_call(cmd, cwd=os.path.dirname(out_path), stderr=subprocess.DEVNULL)


def _kernel(lines: list[str], symbol: str) -> tuple[list[str], int]:
    s = next(i for i, l in enumerate(lines) if l.startswith(symbol + ":"))
    e = next(i for i in range(s, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[s:e], s


def _parse(lines: list[str]):
    """Basic blocks as lists of pre-parsed instructions."""
    blocks, cur = [], []
    for i, l in enumerate(lines):
        t = l.strip()
        m = re.match(r"^(\.LBB\w+):", l)
        if m:
            if cur:
                blocks.append(cur)
            cur = [("label", m.group(1), i)]
            continue
        if not t or t.startswith(";"):
            continue
        cur.append(("ins", t, i))
        if t.startswith(("s_cbranch", "s_branch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    names = {b[0][1]: k for k, b in enumerate(blocks) if b and b[0][0] == "label"}
    parsed = []
    for b in blocks:
        ops = []
        for kind, t, i in b:
            if kind != "ins":
                continue
            op = {"line": i, "text": t}
            m = _WAIT.match(t)
            if m:
                op["wait"] = int(m.group(1))
            m = _LOAD.match(t)
            if m and i > 0 and "s_nop 4" in lines[i - 1]:
                op["asm_load"] = m.group(1)
            op["vmem"] = bool(_VMEM.match(t))
            parts = t.split(None, 1)
            op["name"] = parts[0]
            if len(parts) == 2:
                args = parts[1]
                op["dst"] = args.split(",")[0].strip()
                op["srcs"] = args.split(",", 1)[1] if "," in args else ""
                op["args"] = args
            ops.append(op)
        last = ops[-1]["text"] if ops else ""
        parsed.append((ops, last))
    return parsed, names


def _succ(parsed, names, k):
    last = parsed[k][1]
    if last.startswith("s_branch"):
        return [names[last.split()[1]]]
    if last.startswith(("s_endpgm", "s_setpc")):
        return []
    out = [names[last.split()[1]]] if last.startswith("s_cbranch") else []
    if k + 1 < len(parsed):
        out.append(k + 1)
    return out


def check_kernel(lines: list[str], symbol: str):
    """Returns (hazards, refills): (load line, use line, instruction) triples."""
    body, base = _kernel(lines, symbol)
    parsed, names = _parse(body)
    track = set()
    for ops, _ in parsed:
        for op in ops:
            m = _ANDVCC.match(op["text"])
            if m:
                track.add((m.group(2), m.group(3)))
    IN = {(0, ()): {}}
    work = [(0, ())]
    found = set()
    while work:
        node = work.pop()
        k, fl = node
        st = dict(IN[node])
        flags = dict(fl)
        vcc = None
        for op in parsed[k][0]:
            t = op["text"]
            if "wait" in op:
                st = {r: v for r, v in st.items() if v[0] < op["wait"]}
                continue
            if st and "asm_load" not in op and "srcs" in op:
                store = op["name"].startswith(("ds_write", "buffer_store"))
                for r in list(st):
                    pat = r"\b%s\b" % r
                    if re.search(pat, op["srcs"]) or (store and re.search(pat, op["args"])):
                        found.add((st[r][1], op["line"], t))
                    if op["dst"] == r and not store and not op["name"].startswith("s_"):
                        found.add((st[r][1], op["line"], "overwritten by " + t))
            if op["vmem"]:
                st = {r: (min(v[0] + 1, _CAP), v[1]) for r, v in st.items()}
            if "asm_load" in op:
                st[op["asm_load"]] = (0, op["line"])
            m = _MOV64.match(t)
            if m and (m.group(1), m.group(2)) in track:
                flags[(m.group(1), m.group(2))] = int(m.group(3))
                continue
            m = _ANDVCC.match(t)
            if m:
                v = flags.get((m.group(2), m.group(3)))
                vcc = None if v is None else ((v != 0) if m.group(1) == "and" else (v == 0))
                continue
            m = _SWRITE.match(t)
            if m and (m.group(1), m.group(2)) in flags:
                del flags[(m.group(1), m.group(2))]
            if _VCCW.match(t):
                vcc = None
        last = parsed[k][1]
        nxt = _succ(parsed, names, k)
        if vcc is not None and last.startswith(("s_cbranch_vccz", "s_cbranch_vccnz")):
            taken = (not vcc) if last.startswith("s_cbranch_vccz") else vcc
            nxt = [names[last.split()[1]]] if taken else ([k + 1] if k + 1 < len(parsed) else [])
        nfl = tuple(sorted(flags.items()))
        for s in nxt:
            key = (s, nfl)
            old = IN.get(key)
            if old is None:
                IN[key] = dict(st)
                work.append(key)
                continue
            changed = False
            for r, v in st.items():
                if r not in old:
                    old[r] = v
                    changed = True
                elif v[0] < old[r][0]:
                    old[r] = (v[0], old[r][1])
                    changed = True
            if changed:
                work.append(key)
    rel = sorted((a + base + 1, b + base + 1, t) for a, b, t in found)
    hazards = [x for x in rel if not x[2].startswith("ds_write")]
    refills = [x for x in rel if x[2].startswith("ds_write")]
    return hazards, refills


DECODERS = ["_ZN2cg8k_decodeILb%dELb%dEEEvNS_10DecodeArgsE" % (p, b) for p in (0, 1) for b in (0, 1)]


def check_all(asm_path: str | None = None):
    """{kernel symbol: (hazards, refills)} for the four decoder instances."""
    if asm_path is None:
        d = tempfile.mkdtemp(prefix="cg_asm_")
        asm_path = os.path.join(d, "cg_kernels.s")
        compile_asm(asm_path)
    lines = open(asm_path).read().split("\n")
    return {k: check_kernel(lines, k) for k in DECODERS}


if __name__ == "__main__":
    import sys

    res = check_all(sys.argv[1] if len(sys.argv) > 1 else None)
    for k, (hz, rf) in res.items():
        print(k, "hazards", len(hz), "refills", len(rf))
        for h in hz[:8]:
            print("   load line %d, use line %d: %s" % h)
