#!/usr/bin/env python3
"""Benchmark of the gfx950 KV-cache codec on one MI355X.

One step = one pass of the whole hot path over the workload already resident
in HBM: cg_build_tables (quantize + delta + per-channel histograms + 12-bit
tables), cg_encode (interleaved rANS + record compaction) and cg_decode
(fused rANS decode + token prefix + dequantize into the contiguous cache).

value = fp16 bytes of the KV cache / seconds per step (round trip). The JSON
line also carries decode / encode / table-build GB/s, the compression ratio,
the roofline of the dominant kernel and the CPU oracle timed on a sample.

Variants (their own lines, not the headline): --dtype bf16 runs the same
workload as bfloat16 elements (the fp16 draw rounded to bfloat16);
--robust builds robust tables from the first quarter of the tokens only
(calibration data) and encodes the whole cache with them; --attend times
the restore-and-consume step instead: cg_decode_paged of every chunk into a
paged pool, then cg_attend_paged of one new token per layer over it;
--level-mix encodes every chunk at the three quality presets and times
cg_decode of a seeded per-chunk level mix (with --config long: the
80K-token multi-level workload); --stream times the streaming workload
(records from pinned host memory into a paged cache, beside a plain pinned
copy of the same bytes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV decode & encode GB/s (fp16 bytes) on 1 MI355X; % HBM peak; compression ratio"
HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    """The host's CPU model and core counts (the oracle baseline's cores)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu": model, "nproc": os.cpu_count(), "usable": aff}


def _oracle_sample(O, cfg, lvd, Xs, T, dtype, flags, layer):
    """build tables + encode + decode of one layer's sample with the oracle."""
    shp = O.shape(1, cfg.kv_heads, cfg.head_dim, T, cfg.chunk_tokens, dtype)
    steps = [lvd.steps[lvd.layer_group[layer]]]
    blob, _ = O.build_tables(shp, lvd.level_id, [0], steps, Xs, flags=flags)
    data, offs = O.encode_all(shp, blob, Xs)
    O.decode_all(shp, blob, data, offs)


def cpu_baseline(cfg, X, seconds=10.0, dtype=0, flags=0, cores=16):
    """The oracle on a bounded sample of the same workload: one layer, all
    heads, the first two chunks; build + encode + decode. First single-
    threaded (layer 0, repeated for about `seconds`), then the same function
    on `cores` threads at once, each on its own layer (independent units; the
    C oracle runs without the GIL). X: element bits (uint16) of the first
    `cores` layers of the workload."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O

    lvd = cfg.levels[0]
    T = min(cfg.tokens, 2 * cfg.chunk_tokens)
    samples = [np.ascontiguousarray(X[l:l + 1, :, :, :T, :]) for l in range(X.shape[0])]
    elems = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        _oracle_sample(O, cfg, lvd, samples[0], T, dtype, flags, 0)
        elems += samples[0].size
        reps += 1
        if time.perf_counter() - t0 >= seconds or reps >= 50:
            break
    dt = time.perf_counter() - t0
    n = min(cores, len(samples))
    reps_n = max(1, reps // 2)

    def worker(l):
        for _ in range(reps_n):
            _oracle_sample(O, cfg, lvd, samples[l], T, dtype, flags, l)

    t1 = time.perf_counter()
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(worker, range(n)))
    dt_n = time.perf_counter() - t1
    return {"value": round(2 * elems / dt / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "layer 0 of the workload, %d tokens (%d chunks), all heads: build tables + "
                      "encode + decode, %d repetition(s), %.1f s single-threaded" % (
                          T, -(-T // cfg.chunk_tokens), reps, dt),
            "host": host_info(),
            "x_cores": {"value": round(2 * n * reps_n * samples[0].size / dt_n / 1e9, 5), "unit": "GB/s",
                        "cores": n, "sample": "the same function on %d threads at once, thread k on layer k "
                        "(%d repetition(s) each), %.1f s" % (n, reps_n, dt_n)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps first (the clock settles over the first ten or so)")
    ap.add_argument("--config", default="34b", help="tiny | 7b | 34b | long (workload of the step)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-launch HBM bytes of the kernels from rocprofv3 counters")
    ap.add_argument("--dtype", choices=("fp16", "bf16"), default="fp16")
    ap.add_argument("--robust", action="store_true",
                    help="robust tables from the first quarter of the tokens")
    ap.add_argument("--attend", action="store_true",
                    help="time decode into a paged pool + attention over it")
    ap.add_argument("--level-mix", action="store_true",
                    help="time a decode of chunk records of three quality levels mixed per chunk")
    ap.add_argument("--stream", action="store_true",
                    help="the streaming workload: records from pinned host memory decoded into a paged "
                         "cache while the next one is copied, against a plain pinned copy of the same bytes")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed steps, one library copy of this many bytes (the calibration "
                         "launch for the FETCH_SIZE / WRITE_SIZE counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the codec is measured on one GPU only; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_compression_encode_amd import cg as C
    from kv_cache_compression_encode_amd import codec, profiling, synth

    C.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.stream:
        return run_stream(args)
    cfg = synth.CONFIGS[args.config]
    lvd = cfg.levels[0]
    t_gen = time.perf_counter()
    X = synth.generate(cfg)
    log("generated %s %s in %.1f s" % (cfg.name, X.shape, time.perf_counter() - t_gen))
    dev = torch.device("cuda:0")
    x = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.float16)
    bf = args.dtype == "bf16"
    if bf:
        x = x.to(torch.bfloat16)
    N = x.numel()
    fp16_bytes = 2 * N

    dt = C.CG_DTYPE_BF16 if bf else C.CG_DTYPE_F16
    shp = codec.shape_of(cfg, dtype=dt)
    lv = codec.level_of(lvd)
    cd = codec.Codec(shp, dev)
    flags = C.CG_TABLES_ROBUST if args.robust else 0
    if args.robust:
        t_cal = cfg.tokens // 4
        x_tab = x[:, :, :, :t_cal, :].contiguous()
        cd_tab = codec.Codec(codec.shape_of(cfg, tokens=t_cal, dtype=dt), dev)
    else:
        x_tab, cd_tab = x, cd
    nch = codec.n_chunks(shp)
    tables = torch.empty(cd.tables_bytes(lv), dtype=torch.uint8, device=dev)
    out = torch.empty(C.cg_encode_bound(shp, 0, nch), dtype=torch.uint8, device=dev)
    offs = torch.zeros(nch + 1, dtype=torch.int64, device=dev)
    y = torch.empty_like(x)
    refs = torch.empty(nch * C.REF_BYTES, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None, kt=None):
        kt = kt or {}
        if ev:
            ev[0].record(stream)
        cd_tab.build_tables(x_tab, lv, tables=tables, prof=kt.get("build"), flags=flags)
        if ev:
            ev[1].record(stream)
        cd.encode(x, lv, tables, out=out, offsets=offs, prof=kt.get("encode"))
        if ev:
            ev[2].record(stream)
        C.cg_make_refs(out, offs, nch, 0, refs)
        if ev:
            ev[3].record(stream)
        cd.decode([lv], [tables], refs, nch, y=y, prof=kt.get("decode"))
        if ev:
            ev[4].record(stream)

    if args.attend:
        return run_attend(args, cfg, lvd, cd, x, shp, lv, tables, out, offs, refs, nch, stream)
    if args.level_mix:
        return run_level_mix(args, cfg, cd, x, shp, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert cd.read_status() == 0, "codec reported status %d" % cd.read_status()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    timers = [{k: C.KernelTimer() for k in ("build", "encode", "decode")} for _ in range(args.steps)]
    # the per-call and per-kernel events are recorded inside the timed steps
    # (they cost about 0.5 % of a step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k], timers[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = cd.read_status()
    assert st == 0, "codec reported status %d" % st
    # the data's counters (saturated, NaN, escapes) from one more, untimed
    # table build: asking for them selects the counting variant of k_hist
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    cd_tab.build_tables(x_tab, lv, flags=flags, stats=stats)
    torch.cuda.synchronize()
    # achievable HBM bandwidth on this machine: the library's copy kernel over
    # 4 GiB (2 x 4 GiB of traffic), best of 3 (skipped in counter-calibration
    # runs, whose only copy launch is the calibration one)
    cbytes = 0 if args.copy_bytes > 0 else 4 << 30
    csrc = torch.empty(cbytes, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    copy_ms = []
    for _ in range(3 if cbytes else 0):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        C.cg_copy(cdst, csrc, cbytes)
        e1.record(stream)
        e1.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    copy_gbps = 2 * cbytes / (min(copy_ms) / 1e3) / 1e9 if cbytes else None
    del csrc, cdst
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        C.cg_copy(dst, src, args.copy_bytes)
        torch.cuda.synchronize()
        del src, dst

    # per call (all kernels of the call) and per main kernel, mean over the steps
    ms = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in events])
    t_build, t_enc, t_refs, t_dec = ms.mean(axis=0)
    kms = {k: float(np.mean([t[k].elapsed_ms() for t in timers])) for k in ("build", "encode", "decode")}
    comp = int(offs[-1].item())
    fmt = cd.format_bytes(lv)
    ratio = fp16_bytes / comp
    # correctness of this very run: the decoded cache equals numpy's
    # dequant(quant(x)) on sampled (layer, K|V, head) slices
    rng = np.random.default_rng(0)
    bad = 0
    for _ in range(4):
        l, kv, h = int(rng.integers(cfg.layers)), int(rng.integers(2)), int(rng.integers(cfg.kv_heads))
        step_ = np.float32(lvd.steps[lvd.layer_group[l]])
        xs = x[l, kv, h].cpu().to(torch.float64).numpy()
        with np.errstate(all="ignore"):
            q = np.clip(np.rint((xs / np.float64(step_)).astype(np.float32)), -32768, 32767)
            q = np.nan_to_num(q).astype(np.int32)  # an integer code: no signed zero
            r32 = torch.from_numpy(q.astype(np.float32) * step_)
            ref = r32.to(x.dtype).view(torch.int16).numpy().view(np.uint16)
        got = y[l, kv, h].cpu().view(torch.int16).numpy().view(np.uint16)
        bad += int(np.count_nonzero(got != ref))
    assert bad == 0, "decoded values differ from the reference reconstruction"

    # dominant kernel of the step and its roofline
    # algorithmic bytes: the table build reads the cache and writes the
    # tables' format section (512 B per table); the encoder reads the cache
    # and writes the records; the decoder reads the records and the tables
    # and writes the cache
    phases = {
        "k_hist": (kms["build"], 2 * x_tab.numel() + fmt),
        "k_encode": (kms["encode"], fp16_bytes + comp),
        "k_decode": (kms["decode"], fp16_bytes + comp + fmt),
    }
    dom = max(phases, key=lambda k: phases[k][0])
    variant = args.config + ("-bf16" if bf else "") + ("-robust" if args.robust else "")

    def roof(name):
        t, b = phases[name]
        gbps = b / (t / 1e3) / 1e9
        r = {"kernel": name, "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
             "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
             "algorithmic_bytes": int(b), "avg_ms": round(float(t), 4),
             "avg_ms_from": "HIP events on the call's stream around each timed launch",
             "frac_fp16_only": round(fp16_bytes / (t / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
        # counters taken on these very kernel sources and this workload only
        try:
            with open(args.traffic) as f:
                tr = json.load(f).get(variant, {})
            ent = tr.get("kernels", {}).get(name)
            if ent and tr.get("source_hash") == profiling.source_hash():
                r["traffic"] = ent["bytes_per_launch"]
        except (OSError, ValueError):
            pass
        return r

    def roof_alu(name):
        """VALU lane-operations of the kernel (SQ_INSTS_VALU x 64, counted by
        rocprofv3 on these kernel sources) over its measured time, against the
        int32 / non-packed fp32 VALU peak of 256 CUs x 64 lanes x 2.4 GHz."""
        try:
            with open(args.traffic) as f:
                tr = json.load(f).get(variant, {})
            ent = tr.get("sq", {}).get(name)
            if not ent or tr.get("source_hash") != profiling.source_hash():
                return None
        except (OSError, ValueError):
            return None
        ops = ent["SQ_INSTS_VALU"] * 64
        rate = ops / (phases[name][0] / 1e3) / 1e12
        peak = profiling.VALU_PEAK_OPS / 1e12
        return {"kernel": name, "bound": "alu", "achieved": round(rate, 2), "peak": round(peak, 2),
                "unit": "Tops/s", "frac": round(rate / peak, 4), "valu_ops_per_launch": int(ops)}

    res = {
        "metric": METRIC,
        "value": round(fp16_bytes / (wall / args.steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "%s data; fp32 quantize/dequantize, u32 rANS" % args.dtype,
        "data": "synthetic",
        "config": {"workload": "%s: %d layers x %d KV heads x %d dim x %d tokens, %s K+V, chunk %d, "
                               "%s steps %s%s" % (cfg.name, cfg.layers, cfg.kv_heads, cfg.head_dim,
                                                  cfg.tokens, args.dtype, cfg.chunk_tokens, lvd.name,
                                                  "/".join(str(s) for s in lvd.steps),
                                                  ", robust tables from the first %d tokens" % (cfg.tokens // 4)
                                                  if args.robust else ""),
                   "fp16_bytes": fp16_bytes, "chunks": nch},
        "decode_GBps": round(fp16_bytes / (t_dec / 1e3) / 1e9, 1),
        "encode_GBps": round(fp16_bytes / (t_enc / 1e3) / 1e9, 1),
        "build_tables_GBps": round(fp16_bytes / (t_build / 1e3) / 1e9, 1),
        "decode_ms": round(float(t_dec), 4),
        "encode_ms": round(float(t_enc), 4),
        "build_tables_ms": round(float(t_build), 4),
        "compressed_bytes": comp,
        "compression_ratio": round(ratio, 3),
        "compressed_fraction": round(comp / fp16_bytes, 4),
        "ratio_incl_tables": round(fp16_bytes / (comp + fmt), 3),
        "counts": dict(zip(("elements", "saturated", "nan", "escapes"), (int(v) for v in stats.cpu()))),
        # a monitored figure with the pages' health threshold ("CacheGen实战"
        # 3.3: compression ratio above 3:1); the decode's share of the restore
        # latency (under 10 %) is a figure of the streaming line (--stream)
        "monitor": {"compression_ratio": round(ratio, 3), "ratio_healthy_above": 3.0,
                    "decode_share_of_round_trip": round(float(t_dec) / (wall / args.steps * 1e3), 4)},
        "roofline": roof(dom),
        "roofline_decode": roof("k_decode"),
        "roofline_encode": roof("k_encode"),
        "roofline_build": roof("k_hist"),
        "roofline_alu": roof_alu(dom),
        "roofline_alu_decode": roof_alu("k_decode"),
        "roofline_alu_encode": roof_alu("k_encode"),
        "kernel_ms": {"k_hist": round(kms["build"], 4), "k_encode": round(kms["encode"], 4),
                      "k_decode": round(kms["decode"], 4)},
        "copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        "decode_frac_of_copy": round(phases["k_decode"][1] / (phases["k_decode"][0] / 1e3) / 1e9 / copy_gbps, 4)
        if copy_gbps else None,
    }
    if not args.no_cpu_baseline:
        ncores = min(16, host_info()["usable"] or 1, cfg.layers)
        xb = x[:ncores, :, :, :2 * cfg.chunk_tokens].cpu().view(torch.int16).numpy().view(np.uint16)
        res["cpu_baseline"] = cpu_baseline(cfg, xb, args.cpu_seconds, dt, flags, cores=ncores)
    print(json.dumps(res), flush=True)


def run_stream(args):
    """The streaming workload ("CacheGen实战" 2.3: a receive stage, parallel
    GPU decode and a fill stage as a pipeline): the 16K-token 7B-shape cache
    with Student-t innovations is encoded, its 11 records are put in pinned
    host memory, and cg_stream_decode_paged copies each record to the GPU on
    a second stream while the previous one decodes into 16-token pages
    through a seeded random block table. Beside it: a plain pinned
    host-to-device copy of the same bytes (the bound of the pipeline) and the
    decode kernels alone, one record per launch as the pipeline issues them.
    step = one streamed restore of the whole cache; value = restored fp16
    bytes per second."""
    import torch

    from kv_cache_compression_encode_amd import cg as C
    from kv_cache_compression_encode_amd import codec, synth

    cfg = synth.CONFIGS["stream"]
    lvd = cfg.levels[0]
    X = synth.generate(cfg)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.float16)
    shp = codec.shape_of(cfg)
    lv = codec.level_of(lvd)
    cd = codec.Codec(shp, dev)
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    tables = cd.build_tables(x, lv, stats=stats)
    out, offs = cd.encode(x, lv, tables)
    assert cd.read_status() == 0
    fp16_bytes = 2 * x.numel()
    del x
    o = offs.cpu().numpy().astype(np.uint64)
    n = len(o) - 1
    rec_bytes = int(o[-1])
    host = torch.empty(rec_bytes, dtype=torch.uint8).pin_memory()
    host.copy_(out[:rec_bytes].cpu())
    bt = synth.block_table(cfg)
    NB = len(bt)
    btd = torch.from_numpy(bt).to(dev)
    pool = torch.empty((cfg.layers, 2, NB, cfg.kv_heads, 16, cfg.head_dim), dtype=torch.float16, device=dev)
    staging = torch.empty(2 * int(np.diff(o).max()) + 512, dtype=torch.uint8, device=dev)
    refs2 = torch.empty(2 * C.REF_BYTES, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # the bound: one plain pinned host-to-device copy of all record bytes
    dst = torch.empty(rec_bytes, dtype=torch.uint8, device=dev)
    copy_ms = []
    for _ in range(3):
        e0, e1 = ev(), ev()
        e0.record(stream)
        dst.copy_(host, non_blocking=True)
        e1.record(stream)
        e1.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    del dst
    h2d_gbps = rec_bytes / (min(copy_ms) / 1e3) / 1e9

    def streamed():
        C.cg_stream_decode_paged(cd.shp, [lv], [tables], host, o, None, n, staging, refs2, pool, NB, btd,
                                 cd.status, copy_stream=copy_stream)

    for _ in range(args.warmup):
        streamed()
    torch.cuda.synchronize()
    assert cd.read_status() == 0
    evs = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        streamed()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert cd.read_status() == 0
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # the decode kernels alone, one record per launch as the pipeline issues them
    dec_ms = []
    for k in range(n):
        refs, _ = cd.make_refs([(out, offs, [k], 0)])
        kt = C.KernelTimer()
        cd.decode_paged([lv], [tables], refs, 1, pool, btd, prof=kt)
        torch.cuda.synchronize()
        dec_ms.append(kt.elapsed_ms())
    assert cd.read_status() == 0
    ratio = fp16_bytes / rec_bytes
    res = {
        "metric": METRIC,
        "value": round(fp16_bytes / (wall / args.steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 data; fp32 dequantize, u32 rANS",
        "data": "synthetic",
        "config": {"workload": "stream: %d layers x %d KV heads x %d dim x %d tokens, fp16 K+V, Student-t(3) "
                               "innovations, chunk %d, %s steps %s; %d records streamed from pinned host memory "
                               "into 16-token pages of a seeded random block table" % (
                                   cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens,
                                   lvd.name, "/".join(str(v) for v in lvd.steps), n),
                   "fp16_bytes": fp16_bytes, "record_bytes": rec_bytes, "records": n},
        "stream_ms": round(step_ms, 3),
        "records_GBps": round(rec_bytes / (step_ms / 1e3) / 1e9, 2),
        "h2d_copy_GBps": round(h2d_gbps, 2),
        "frac_of_h2d_copy": round(rec_bytes / (step_ms / 1e3) / 1e9 / h2d_gbps, 4),
        "decode_kernels_ms": round(float(np.sum(dec_ms)), 3),
        "compression_ratio": round(ratio, 3),
        "counts": dict(zip(("elements", "saturated", "nan", "escapes"), (int(v) for v in stats.cpu()))),
        # the pages' monitored figures ("CacheGen实战" 3.3): decode latency
        # under 10 % of the total, compression ratio above 3:1. The decode
        # runs under the next record's copy, so the latency it adds to the
        # restore is the streamed time beyond a plain copy of the same bytes;
        # the kernels' own time is given beside it
        "monitor": {"compression_ratio": round(ratio, 3), "ratio_healthy_above": 3.0,
                    "decode_latency_share": round(max(0.0, step_ms - rec_bytes / h2d_gbps / 1e6) / step_ms, 4),
                    "decode_share_healthy_below": 0.10,
                    "decode_kernels_share": round(float(np.sum(dec_ms)) / step_ms, 4)},
    }
    print(json.dumps(res), flush=True)


def run_level_mix(args, cfg, cd, x, shp, stream):
    """Every chunk encoded at the three quality levels ("CacheGen实战" 2.1 and
    3.1: high 0.3/0.8/1.2, balanced 0.5/1.0/1.5, fast 0.8/1.5/2.0 over thirds
    of the layers), then one cg_decode of the records of a per-chunk level mix
    drawn from the seed. Step = that decode with the references in chunk
    order (levels interleaved); the same records referenced in runs of one
    level are timed beside it. The two orders alternate, two turns each of
    `steps` decodes; "steps" counts the timed decodes of the interleaved
    order."""
    import numpy as np
    import torch

    from kv_cache_compression_encode_amd import cg as C
    from kv_cache_compression_encode_amd import codec, synth

    dev = x.device
    nch = codec.n_chunks(shp)
    presets = synth.CONFIGS["long"].levels  # the same 48-layer groups
    assert len(presets[0].layer_group) == cfg.layers
    lvs = [codec.level_of(p) for p in presets]
    tabs, outs, ratios = [], [], []
    for lv in lvs:
        t = cd.build_tables(x, lv)
        out, offs = cd.encode(x, lv, t)
        tabs.append(t)
        outs.append((out, offs))
    torch.cuda.synchronize()
    assert cd.read_status() == 0
    fp16_bytes = 2 * x.numel()
    for out, offs in outs:
        ratios.append(round(fp16_bytes / int(offs[-1].item()), 3))
    mix = np.random.default_rng([0, cfg.config_id, 999]).integers(0, len(lvs), nch)
    order_mixed = list(range(nch))
    order_runs = sorted(range(nch), key=lambda c: (int(mix[c]), c))
    refs = {}
    for name, order in (("mixed", order_mixed), ("runs", order_runs)):
        refs[name] = cd.make_refs([(outs[int(mix[c])][0], outs[int(mix[c])][1], [c], int(mix[c])) for c in order])
    y = torch.empty_like(x)
    comp = sum(int((outs[int(mix[c])][1][c + 1] - outs[int(mix[c])][1][c]).item()) for c in range(nch))

    def timed(name):
        r, n = refs[name]
        for _ in range(args.warmup):
            cd.decode(lvs, tabs, r, n, y=y)
        torch.cuda.synchronize()
        assert cd.read_status() == 0
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        kt = [C.KernelTimer() for _ in range(args.steps)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for k in range(args.steps):
            cd.decode(lvs, tabs, r, n, y=y, prof=kt[k])
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        assert cd.read_status() == 0
        call = float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]))
        return wall, call, float(np.mean([t.elapsed_ms() for t in kt]))

    # the two orders alternate (twice each), so neither gets the warmer or
    # cooler part of the run
    res_o = {"runs": [], "mixed": []}
    for name in ("runs", "mixed", "runs", "mixed"):
        res_o[name].append(timed(name))
    wall, call, kern = (float(np.mean(v)) for v in zip(*res_o["mixed"]))
    wall_r, call_r, kern_r = (float(np.mean(v)) for v in zip(*res_o["runs"]))
    # correctness of this run: sampled (layer, K|V, head) slices against
    # numpy's dequant(quant(x)) with each chunk's own level
    rng = np.random.default_rng(2)
    for _ in range(4):
        l, kv, h = int(rng.integers(cfg.layers)), int(rng.integers(2)), int(rng.integers(cfg.kv_heads))
        xs = x[l, kv, h].cpu().to(torch.float64).numpy()
        got = y[l, kv, h].cpu().view(torch.int16).numpy().view(np.uint16)
        for c in range(nch):
            p = presets[int(mix[c])]
            st = np.float32(p.steps[p.layer_group[l]])
            rows = slice(c * cfg.chunk_tokens, min((c + 1) * cfg.chunk_tokens, cfg.tokens))
            with np.errstate(all="ignore"):
                q = np.clip(np.rint((xs[rows] / np.float64(st)).astype(np.float32)), -32768, 32767)
                q = np.nan_to_num(q).astype(np.int32)
                ref = torch.from_numpy(q.astype(np.float32) * st).to(x.dtype).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(got[rows], ref), (l, kv, h, c)
    # the method's bytes: fp16 out, records in, each level's tables' format
    # section (512 B per table), as in the round-trip line
    n_tables = sum(2 * lv.n_groups * cfg.kv_heads * cfg.head_dim for lv in lvs)
    dec_bytes = fp16_bytes + comp + n_tables * 512
    gbps = dec_bytes / (kern / 1e3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(fp16_bytes / (wall / args.steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": 2 * args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "%s data; fp32 dequantize, u32 rANS" % args.dtype,
        "data": "synthetic",
        "config": {"workload": "%s level mix: %d layers x %d KV heads x %d dim x %d tokens, chunk %d, each "
                               "chunk encoded at high/balanced/fast, decoded at a seeded per-chunk mix "
                               "(%s)" % (cfg.name, cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens,
                                         cfg.chunk_tokens, "".join("hbf"[int(m)] for m in mix)),
                   "fp16_bytes": fp16_bytes, "chunks": nch},
        "decode_ms": round(call, 4),
        "decode_GBps": round(fp16_bytes / (call / 1e3) / 1e9, 1),
        "decode_runs_ms": round(call_r, 4),
        "decode_runs_GBps": round(fp16_bytes / (call_r / 1e3) / 1e9, 1),
        "ratio_per_level": dict(zip(("high", "balanced", "fast"), ratios)),
        "compressed_bytes_mixed": comp,
        "roofline": {"kernel": "k_decode", "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes": int(dec_bytes), "avg_ms": round(kern, 4)},
        "kernel_ms": {"k_decode_mixed": round(kern, 4), "k_decode_runs": round(kern_r, 4)},
    }
    print(json.dumps(res), flush=True)


# query heads per kv head of the models the workloads are shaped after
# (34B: 64 query heads over 8 kv heads; 7B: 32 over 32)
Q_HEADS = {"tiny": 4, "7b": 32, "34b": 64, "long": 64, "stream": 32}


def run_attend(args, cfg, lvd, cd, x, shp, lv, tables, out, offs, refs, nch, stream):
    """Step = cg_decode_paged of every chunk into a paged pool (random block
    placement) + cg_attend_paged of one new token per layer over the pool."""
    import numpy as np
    import torch

    from kv_cache_compression_encode_amd import cg as C
    from kv_cache_compression_encode_amd import profiling

    dev = x.device
    cd.build_tables(x, lv, tables=tables)
    cd.encode(x, lv, tables, out=out, offsets=offs)
    C.cg_make_refs(out, offs, nch, 0, refs)
    torch.cuda.synchronize()
    assert cd.read_status() == 0
    nbl = -(-cfg.tokens // 16)
    bt = torch.from_numpy(np.random.default_rng([0, cfg.config_id, 998]).permutation(nbl).astype(np.int32)).to(dev)
    del x
    from kv_cache_compression_encode_amd.codec import torch_dtype
    pool = torch.empty((cfg.layers, 2, nbl, cfg.kv_heads, 16, cfg.head_dim), dtype=torch_dtype(shp), device=dev)
    Hq = Q_HEADS[cfg.name]
    g = torch.Generator(device="cpu").manual_seed(7)
    q = torch.randn((cfg.layers, Hq, cfg.head_dim), generator=g).to(torch_dtype(shp)).to(dev)
    o = torch.empty((cfg.layers, Hq, cfg.head_dim), dtype=torch.float32, device=dev)
    scale = 1.0 / float(np.sqrt(cfg.head_dim))

    def step(ev=None, kt=None):
        kt = kt or {}
        if ev:
            ev[0].record(stream)
        cd.decode_paged([lv], [tables], refs, nch, pool, bt, prof=kt.get("decode"))
        if ev:
            ev[1].record(stream)
        cd.attend_paged(q, pool, bt, cfg.tokens, scale, o=o, prof=kt.get("attend"))
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert cd.read_status() == 0
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    timers = [{k: C.KernelTimer() for k in ("decode", "attend")} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k], timers[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert cd.read_status() == 0
    if args.copy_bytes > 0:  # calibration launch for the counter runs
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        C.cg_copy(torch.empty_like(src), src, args.copy_bytes)
        torch.cuda.synchronize()
        del src
    ms = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(2)] for e in events])
    t_dec, t_att = ms.mean(axis=0)
    kms = {k: float(np.mean([t[k].elapsed_ms() for t in timers])) for k in ("decode", "attend")}
    kv_bytes = 2 * cfg.n_elements
    comp = int(offs[-1].item())
    ws = C.cg_attend_workspace_bytes(shp, Hq, cfg.tokens)
    # k_attend reads K and V once, q once, and writes its partials
    att_bytes = kv_bytes + q.numel() * 2 + ws
    # correctness of this run: sampled (layer, query head) against the same
    # definition in float64 on the host, within the bound the tests use
    rng = np.random.default_rng(1)
    G = Hq // cfg.kv_heads
    tdt = torch_dtype(shp)
    worst = 0.0
    for _ in range(3):
        l, qh = int(rng.integers(cfg.layers)), int(rng.integers(Hq))
        h = qh // G
        K = pool[l, 0][bt.long(), h].reshape(-1, cfg.head_dim).to(torch.float64).cpu().numpy()
        V = pool[l, 1][bt.long(), h].reshape(-1, cfg.head_dim).to(torch.float64).cpu().numpy()
        qv = q[l, qh].to(torch.float64).cpu().numpy()
        sc = scale * (K @ qv)
        p = np.exp(sc - sc.max())
        ref = (p @ V) / p.sum()
        tol = np.abs(V).max() * (4 * scale * cfg.head_dim * 2.0**-24 * np.abs(K * qv).sum(axis=1).max() + 1e-4)
        err = float(np.abs(o[l, qh].cpu().numpy().astype(np.float64) - ref).max())
        assert err <= tol, (l, qh, err, tol)
        worst = max(worst, err / tol)
    gbps = att_bytes / (kms["attend"] / 1e3) / 1e9
    roof = {"kernel": "k_attend", "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
            "algorithmic_bytes": int(att_bytes), "avg_ms": round(kms["attend"], 4)}
    variant = args.config + ("-bf16" if shp.dtype == C.CG_DTYPE_BF16 else "") + "-attend"
    try:
        with open(args.traffic) as f:
            tr = json.load(f).get(variant, {})
        ent = tr.get("kernels", {}).get("k_attend")
        if ent and tr.get("source_hash") == profiling.source_hash():
            roof["traffic"] = ent["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    res = {
        "metric": METRIC,
        "value": round(kv_bytes / (wall / args.steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "%s data; fp32 softmax and P.V, MFMA %s scores" % (args.dtype, args.dtype),
        "data": "synthetic",
        "config": {"workload": "%s restore + attend: decode %d chunk records into a paged pool (16-token "
                               "blocks, random placement), then one new token per layer, %d query heads over "
                               "%d kv heads x %d tokens" % (cfg.name, nch, Hq, cfg.kv_heads, cfg.tokens),
                   "kv_bytes": kv_bytes, "compressed_bytes": comp},
        "decode_paged_ms": round(float(t_dec), 4),
        "attend_ms": round(float(t_att), 4),
        "kernel_ms": {"k_decode_paged": round(kms["decode"], 4), "k_attend": round(kms["attend"], 4)},
        "attend_GBps": round(gbps, 1),
        "roofline": roof,
        "attend_err_over_bound": round(worst, 4),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
