"""Summaries of rocprofv3 output for the repository's profiles/ directory.

- ``stats``: per-kernel call counts and durations from a
  ``rocprofv3 --kernel-trace --stats -f csv`` run, as a markdown table.
- ``traffic``: HBM bytes per launch of the codec kernels from two
  ``rocprofv3 --pmc`` runs (FETCH_SIZE, then WRITE_SIZE, both KiB per
  dispatch), each scaled by what the same counter reads for the library's
  plain copy kernel (k_copy) moving a known number of bytes. Written as JSON
  (read by bench.py) and as markdown.

- ``stall``: where the waves' time goes per kernel (waiting at s_waitcnt,
  issuing scalar ALU, LDS or other instructions) from two SQ counter passes
  over the same workload, as markdown.

All record the source hash of the kernels they describe; bench.py reports
the traffic only while the kernel sources still have that hash.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ("csrc/cg_kernels.hip", "csrc/cg_layout.h", "csrc/cg_api.cpp")
# kernel symbol fragment -> short name used by bench.py
# (the codec kernels are templates on the element type; one run uses one type)
KERNELS = {"k_hist": "cg::k_hist<", "k_encode": "cg::k_encode<", "k_decode": "cg::k_decode<false,",
           "k_decode_paged": "cg::k_decode<true,", "k_write": "cg::k_write(", "k_copy": "cg::k_copy(",
           "k_attend": "cg::k_attend<"}


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    found = sorted(glob.glob(pattern, recursive=True))
    if not found:
        raise FileNotFoundError(pattern)
    return found[0]


def kernel_stats(run_dir: str):
    """[(name, calls, average us, total ms, percent)] from *_kernel_stats.csv."""
    rows = []
    with open(_one(os.path.join(run_dir, "**", "*kernel_stats.csv"))) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    rows.sort(key=lambda r: -r[3])
    return rows


def kernel_trace(run_dir: str):
    """Kernel name -> durations in microseconds, in dispatch order, from
    *_kernel_trace.csv."""
    per = {}
    with open(_one(os.path.join(run_dir, "**", "*kernel_trace.csv"))) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return per


def timed_average(run_dir: str, skip: int, count: int = 0):
    """Short kernel name -> (launches, mean us) over each codec kernel's
    launches after its first `skip` (the benchmark's warm-up steps); with
    count > 0 only the `count` launches after those (the timed steps, not an
    untimed launch the benchmark makes afterwards)."""
    out = {}
    for name, d in kernel_trace(run_dir).items():
        for short, frag in KERNELS.items():
            if frag in name and len(d) > skip:
                t = d[skip:skip + count] if count > 0 else d[skip:]
                out[short] = (len(t), sum(t) / len(t))
    return out


def counter_per_kernel(run_dir: str, counter: str):
    """short kernel name -> counter value of the kernel's first dispatch (KiB
    for the size counters), from *_counter_collection.csv. The counter runs
    time one step without warm-up, so the first dispatch of each codec
    kernel is the step's; a later one is bench.py's untimed counting build
    (a k_hist variant with more work) or its copy."""
    vals = {}
    with open(_one(os.path.join(run_dir, "**", "*counter_collection.csv"))) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            for short, frag in KERNELS.items():
                if frag in r["Kernel_Name"]:
                    vals.setdefault(short, []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: min(v)[1] for k, v in vals.items()}


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int):
    fetch = counter_per_kernel(fetch_dir, "FETCH_SIZE")
    write = counter_per_kernel(write_dir, "WRITE_SIZE")
    if "k_copy" not in fetch or "k_copy" not in write:
        raise ValueError("the runs hold no k_copy dispatch to calibrate against")
    f_fetch = copy_bytes / (fetch["k_copy"] * 1024.0)
    f_write = copy_bytes / (write["k_copy"] * 1024.0)
    out = {"copy_bytes": copy_bytes, "fetch_factor": round(f_fetch, 5), "write_factor": round(f_write, 5),
           "kernels": {}}
    for k in sorted(set(fetch) & set(write)):
        rb = fetch[k] * 1024.0 * f_fetch
        wb = write[k] * 1024.0 * f_write
        out["kernels"][k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                             "read_bytes": int(rb), "write_bytes": int(wb), "bytes_per_launch": int(rb + wb)}
    return out


SQ_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_ANY")
# int32 / non-packed fp32 VALU lane operations per second: 256 CUs x 4 SIMDs x
# 16 lanes x 2.4 GHz (= 157.3 TFLOP/s fp32 / 2 for FMA / 2 for packed issue)
VALU_PEAK_OPS = 256 * 4 * 16 * 2.4e9


def sq(sq_dir: str, trace_dir: str, skip: int = 2, count: int = 5):
    """Per kernel: SQ counters of one dispatch and, with the kernel trace's
    average over the timed launches (after `skip` warm-ups, `count` of
    them), the achieved VALU lane-operation rate."""
    per = {c: counter_per_kernel(sq_dir, c) for c in SQ_COUNTERS}
    dur = {k: us for k, (n, us) in timed_average(trace_dir, skip, count).items()}
    out = {}
    for k in per["SQ_INSTS_VALU"]:
        e = {c: per[c].get(k) for c in SQ_COUNTERS}
        if k in dur:
            e["avg_us"] = dur[k]
            e["valu_lane_ops_per_s"] = e["SQ_INSTS_VALU"] * 64 / (dur[k] * 1e-6)
            e["valu_frac"] = e["valu_lane_ops_per_s"] / VALU_PEAK_OPS
        out[k] = e
    return out


STALL_A = ("SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
           "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC")
STALL_B = ("SQ_INSTS_VALU", "SQ_LDS_DATA_FIFO_FULL")


def stall(a_dir: str, b_dir: str):
    """Per kernel: fractions of the waves' lifetimes (SQ_WAVE_CYCLES) spent
    waiting at s_waitcnt, waiting to issue LDS instructions, issuing any,
    scalar-ALU or other sequencer instructions (mean per dispatch)."""
    per = {c: counter_per_kernel(a_dir, c) for c in STALL_A}
    per.update({c: counter_per_kernel(b_dir, c) for c in STALL_B})
    out = {}
    for k, wc in per["SQ_WAVE_CYCLES"].items():
        if not wc or k == "k_copy":
            continue
        out[k] = {"wave_cycles": 4 * wc, "wait": per["SQ_WAIT_INST_ANY"][k] / wc,
                  "wait_lds": per["SQ_WAIT_INST_LDS"][k] / wc, "issue": per["SQ_ACTIVE_INST_ANY"][k] / wc,
                  "scalar": per["SQ_ACTIVE_INST_SCA"][k] / wc, "misc": per["SQ_ACTIVE_INST_MISC"][k] / wc,
                  "valu_insts": per["SQ_INSTS_VALU"].get(k, 0.0),
                  "lds_fifo_full": per["SQ_LDS_DATA_FIFO_FULL"].get(k, 0.0)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("run_dir")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True, help="the command that produced run_dir")
    s.add_argument("--note", default="")
    s.add_argument("--skip", type=int, default=0,
                   help="warm-up launches per codec kernel left out of the timed-launch averages")
    s.add_argument("--bench-json", default="",
                   help="the JSON line bench.py printed in the same run (its event-timed kernel averages)")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True, help="output dir of the FETCH_SIZE run")
    t.add_argument("--write", required=True, help="output dir of the WRITE_SIZE run")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--config", required=True, help="workload name the runs used")
    t.add_argument("--command", required=True, help="the two commands, ';'-separated")
    t.add_argument("--json", required=True, help="traffic JSON (merged per workload)")
    t.add_argument("--md", required=True)
    w = sub.add_parser("stall")
    w.add_argument("--a", required=True, help="output dir of the first stall counter pass")
    w.add_argument("--b", required=True, help="output dir of the second stall counter pass")
    w.add_argument("--config", required=True)
    w.add_argument("--command", required=True, help="the commands, ';'-separated lines")
    w.add_argument("--md", required=True)
    q = sub.add_parser("sq")
    q.add_argument("--sq", required=True, help="output dir of the SQ counter run")
    q.add_argument("--trace", required=True, help="output dir of a kernel-trace run of the same sources")
    q.add_argument("--config", required=True)
    q.add_argument("--command", required=True, help="the command, ';'-separated lines")
    q.add_argument("--json", required=True)
    q.add_argument("--md", required=True)
    q.add_argument("--skip", type=int, default=2, help="warm-up launches of the kernel-trace run")
    q.add_argument("--count", type=int, default=5, help="timed launches of the kernel-trace run")
    a = ap.parse_args()
    if a.cmd == "stall":
        res = stall(a.a, a.b)
        with open(a.md, "w") as f:
            f.write("# Wave stall counters per launch, %s workload (rocprofv3)\n\n" % a.config)
            f.write("Kernel sources: hash `%s`. SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_* count in "
                    "units of 4 cycles summed over waves; the fractions are of the waves' lifetimes "
                    "(SQ_WAVE_CYCLES). Waiting: at an s_waitcnt; LDS issue: waiting to issue an LDS "
                    "instruction; scalar: issuing scalar ALU; misc: branches and other sequencer "
                    "instructions. Two counter passes (at most 8 SQ counters each) over the same "
                    "one-step run; the first dispatch of each kernel (the step's).\n\n" % source_hash())
            f.write("Commands (repository root):\n\n```\n%s\n```\n\n" % a.command.replace(";", "\n"))
            f.write("| kernel | waves' cycles | waiting (s_waitcnt) | waiting to issue LDS | issuing any | "
                    "issuing scalar ALU | branches/misc | VALU insts | LDS data FIFO full |\n"
                    "|---|---|---|---|---|---|---|---|---|\n")
            for k in ("k_decode", "k_encode", "k_hist", "k_write", "k_decode_paged", "k_attend"):
                if k not in res:
                    continue
                e = res[k]
                f.write("| %s | %.4g | %.1f %% | %.1f %% | %.1f %% | %.1f %% | %.1f %% | %.4g | %d |\n" % (
                    k, e["wave_cycles"], 100 * e["wait"], 100 * e["wait_lds"], 100 * e["issue"],
                    100 * e["scalar"], 100 * e["misc"], e["valu_insts"], e["lds_fifo_full"]))
        print("wrote", a.md)
        return
    if a.cmd == "sq":
        res = sq(a.sq, a.trace, skip=a.skip, count=a.count)
        doc = {}
        if os.path.exists(a.json):
            with open(a.json) as f:
                doc = json.load(f)
        ent = doc.setdefault(a.config, {})
        if ent.get("source_hash") not in (None, source_hash()):
            ent.clear()
        ent["source_hash"] = source_hash()
        ent["sq"] = res
        with open(a.json, "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
        with open(a.md, "w") as f:
            f.write("# SQ counters per launch, %s workload (rocprofv3)\n\n" % a.config)
            f.write("Kernel sources: hash `%s`. VALU peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = %.2f T "
                    "lane-ops/s (int32 / non-packed fp32). Counters: the first dispatch of each kernel (the one timed step). Durations: the kernel-trace run's timed launches (after %d warm-up steps, the %d timed steps).\n\n"
                    % (source_hash(), VALU_PEAK_OPS / 1e12, a.skip, a.count))
            f.write("Commands (repository root):\n\n```\n%s\n```\n\n" % a.command.replace(";", "\n"))
            f.write("| kernel | avg us | waves | VALU insts | SALU insts | LDS insts | VALU lane-ops/s | of VALU "
                    "peak | LDS bank conflicts | wait-any / wave-busy |\n|---|---|---|---|---|---|---|---|---|---|\n")
            for k, e in sorted(res.items()):
                if "avg_us" not in e:
                    continue
                f.write("| %s | %.1f | %d | %.4g | %.4g | %.4g | %.2f T | %.1f %% | %d | %.4g |\n" % (
                    k, e["avg_us"], e["SQ_WAVES"], e["SQ_INSTS_VALU"], e["SQ_INSTS_SALU"], e["SQ_INSTS_LDS"],
                    e["valu_lane_ops_per_s"] / 1e12, 100 * e["valu_frac"], e["SQ_LDS_BANK_CONFLICT"] or 0,
                    e["SQ_WAIT_ANY"] or 0))
        print("wrote", a.json, a.md)
        return
    if a.cmd == "stats":
        rows = kernel_stats(a.run_dir)
        with open(a.out, "w") as f:
            f.write("# %s\n\n" % a.title)
            if a.note:
                f.write(a.note + "\n\n")
            f.write("Kernel sources: hash `%s`.\n\nCommand (repository root):\n\n```\n%s\n```\n\n"
                    % (source_hash(), a.command))
            f.write("| kernel | calls | average us | total ms | % |\n|---|---|---|---|---|\n")
            for name, calls, avg, tot, pct in rows:
                f.write("| `%s` | %d | %.1f | %.2f | %.2f |\n" % (name[:90], calls, avg, tot, pct))
            if a.skip:
                bench, steps = {}, 0
                if a.bench_json:
                    with open(a.bench_json) as bj:
                        line = [ln for ln in bj.read().splitlines() if ln.startswith("{")][-1]
                    bj_doc = json.loads(line)
                    bench = bj_doc.get("kernel_ms", {})
                    steps = int(bj_doc.get("steps", 0))
                ta = timed_average(a.run_dir, a.skip, steps)
                f.write("\nTimed launches only (each codec kernel's first %d launches, the warm-up steps, left "
                        "out%s), from the per-dispatch trace%s:\n\n" % (
                            a.skip, ", and only the next %d, the timed steps" % steps if steps else "",
                            ", beside the HIP-event averages bench.py printed in the same run"
                            if bench else ""))
                f.write("| kernel | timed launches | trace average us | bench.py events us | trace / events |\n"
                        "|---|---|---|---|---|\n")
                for k, (nl, us) in sorted(ta.items()):
                    ev = bench.get(k)
                    f.write("| %s | %d | %.1f | %s | %s |\n" % (
                        k, nl, us, "%.1f" % (1e3 * ev) if ev else "-",
                        "%.3f" % (us / (1e3 * ev)) if ev else "-"))
        print("wrote", a.out)
    else:
        tr = traffic(a.fetch, a.write, a.copy_bytes)
        doc = {}
        if os.path.exists(a.json):
            with open(a.json) as f:
                doc = json.load(f)
        prev = doc.get(a.config, {})
        keep = {"sq": prev["sq"]} if prev.get("source_hash") == source_hash() and "sq" in prev else {}
        doc[a.config] = dict(tr, source_hash=source_hash(), **keep)
        with open(a.json, "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
        with open(a.md, "w") as f:
            f.write("# HBM traffic per launch, %s workload (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n" % a.config)
            f.write("Kernel sources: hash `%s`. Calibration: k_copy reads and writes %d bytes; calibrated "
                    "bytes = counter KiB x 1024 x factor, with factor %.4f for FETCH_SIZE and %.4f for "
                    "WRITE_SIZE (the copy's known bytes over its counter reading).\n\n"
                    % (source_hash(), a.copy_bytes, tr["fetch_factor"], tr["write_factor"]))
            f.write("Commands (repository root):\n\n```\n%s\n```\n\n" % a.command.replace(";", "\n"))
            f.write("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (calibrated) | written bytes "
                    "(calibrated) | total per launch |\n|---|---|---|---|---|---|\n")
            for k, v in tr["kernels"].items():
                f.write("| %s | %.1f | %.1f | %d | %d | %d |\n" % (k, v["fetch_kib"], v["write_kib"],
                                                                  v["read_bytes"], v["write_bytes"],
                                                                  v["bytes_per_launch"]))
        print("wrote", a.json, a.md)


if __name__ == "__main__":
    main()
