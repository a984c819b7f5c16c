"""Full-size workloads through the C ABI, in the launch configuration the
benchmark times, checked on sampled outputs the oracle computes one by one."""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth

from tests import fullsize as F
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
torch = U.torch
C = U.C


def run_level(cd, x, lvd):
    lv = U.codec.level_of(lvd)
    tables = cd.build_tables(x, lv)
    out, offs = cd.encode(x, lv, tables)
    assert cd.read_status() == 0
    used = int(offs[-1])
    out = out[:used].clone()  # release the worst-case allocation
    return lv, tables, out, offs


@pytest.mark.parametrize("name", ["7b", "34b"])
def test_contiguous_roundtrip(name):
    U.need_gpu()
    cfg = synth.CONFIGS[name]
    lvd = cfg.levels[0]
    X = synth.generate(cfg)
    print("generated", name, flush=True)
    cd = U.codec.Codec(U.codec.shape_of(cfg))
    x = U.to_dev(X)
    lv, tables, out, offs = run_level(cd, x, lvd)
    refs, n = cd.refs_for(out, offs)
    y = cd.decode([lv], [tables], refs, n)
    assert cd.read_status() == 0
    rng = np.random.default_rng(1)
    blob = U.u8(tables[:cd.format_bytes(lv)])
    o = offs.cpu().numpy()
    F.check_tables(cfg, lvd, X, blob, rng)
    F.check_groups(cfg, X, blob, lambda a, b: U.u8(out[a:b]), o, rng)
    steps = [lvd.steps[g] for g in lvd.layer_group]
    F.check_slices(cfg, steps, X, lambda l, kv, h: y[l, kv, h].cpu().numpy().view(np.uint16), rng)
    ratio = X.nbytes / int(o[-1])
    print("%s ratio %.3f:1" % (name, ratio), flush=True)
    assert 2.0 < ratio < 20.0


def test_long_context_three_levels_mixed():
    U.need_gpu()
    cfg = synth.CONFIGS["long"]
    X = synth.generate(cfg)
    print("generated long", flush=True)
    cd = U.codec.Codec(U.codec.shape_of(cfg))
    x = U.to_dev(X)
    lvs, tabs, outs = [], [], []
    rng = np.random.default_rng(2)
    for k, lvd in enumerate(cfg.levels):
        lv, tables, out, offs = run_level(cd, x, lvd)
        blob = U.u8(tables[:cd.format_bytes(lv)])
        F.check_tables(cfg, lvd, X, blob, rng, n=3)
        F.check_groups(cfg, X, blob, lambda a, b, out=out: U.u8(out[a:b]), offs.cpu().numpy(), rng, n=2)
        print("level", lvd.name, "ratio %.3f" % (X.nbytes / int(offs[-1])), flush=True)
        lvs.append(lv)
        tabs.append(tables)
        outs.append((out, offs))
    mix = synth.level_mix(cfg)
    parts = [(outs[int(m)][0], outs[int(m)][1], [c], int(m)) for c, m in enumerate(mix)]
    refs, n = cd.make_refs(parts)
    y = cd.decode(lvs, tabs, refs, n)
    assert cd.read_status() == 0
    # per chunk the reconstruction uses that chunk's level
    for _ in range(3):
        c = int(rng.integers(cfg.n_chunks))
        lvd = cfg.levels[int(mix[c])]
        steps = [lvd.steps[g] for g in lvd.layer_group]
        t = slice(c * cfg.chunk_tokens, min((c + 1) * cfg.chunk_tokens, cfg.tokens))
        F.check_slices(cfg, steps, X, lambda l, kv, h: y[l, kv, h].cpu().numpy().view(np.uint16), rng,
                       n=2, tokens=t)


def test_stream_paged():
    U.need_gpu()
    cfg = synth.CONFIGS["stream"]
    lvd = cfg.levels[0]
    X = synth.generate(cfg)
    print("generated stream", flush=True)
    cd = U.codec.Codec(U.codec.shape_of(cfg))
    x = U.to_dev(X)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    lv = U.codec.level_of(lvd)
    tables = cd.build_tables(x, lv, stats=stats)
    out, offs = cd.encode(x, lv, tables)
    assert cd.read_status() == 0
    esc = int(stats[3])
    print("escapes", esc, "per element %.2e" % (esc / x.numel()), flush=True)
    assert esc > 0  # Student-t innovations produce escapes
    bt = synth.block_table(cfg)
    NB = len(bt)
    del x
    pool = torch.empty((cfg.layers, 2, NB, cfg.kv_heads, 16, cfg.head_dim), dtype=torch.float16,
                       device="cuda")
    refs, n = cd.refs_for(out, offs)
    cd.decode_paged([lv], [tables], refs, n, pool, torch.from_numpy(bt).cuda())
    assert cd.read_status() == 0
    rng = np.random.default_rng(3)
    steps = [lvd.steps[g] for g in lvd.layer_group]

    def y_slice(l, kv, h):
        blocks = pool[l, kv, torch.from_numpy(bt.astype(np.int64)).cuda(), h]  # [T/16][16][D]
        return blocks.reshape(cfg.tokens, cfg.head_dim).cpu().numpy().view(np.uint16)

    F.check_slices(cfg, steps, X, y_slice, rng)
    blob = U.u8(tables[:cd.format_bytes(lv)])
    o = offs.cpu().numpy()
    F.check_groups(cfg, X, blob, lambda a, b: U.u8(out[a:b]), o, rng, n=3)

    # the same records streamed from pinned host memory into a second pool
    host = torch.empty(int(o[-1]), dtype=torch.uint8).pin_memory()
    host.copy_(out[:int(o[-1])].cpu())
    staging = torch.empty(2 * int(np.diff(o).max()) + 512, dtype=torch.uint8, device="cuda")
    refs2 = torch.empty(2 * C.REF_BYTES, dtype=torch.uint8, device="cuda")
    pool2 = torch.empty_like(pool)
    copy_stream = torch.cuda.Stream()
    btd = torch.from_numpy(bt).cuda()
    # twice: the first call also pays the copy stream's first use
    for turn in ("first call", "second call"):
        pool2.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        C.cg_stream_decode_paged(cd.shp, [lv], [tables], host, o.astype(np.uint64), None, n, staging, refs2,
                                 pool2, NB, btd, cd.status, copy_stream=copy_stream)
        e1.record()
        assert cd.read_status() == 0
        ms = e0.elapsed_time(e1)
        print("%s: streamed %d records, %.1f MB in %.2f ms (%.1f GB/s host-to-device incl. decode)" % (
            turn, n, o[-1] / 1e6, ms, o[-1] / ms / 1e6), flush=True)
        assert torch.equal(pool2.view(torch.int16), pool.view(torch.int16))


def test_34b_bf16_robust_calibration_tables():
    """The 34B workload as bfloat16 with robust tables built from its first
    quarter of tokens only (calibration data), every chunk encoded with them:
    sampled tables, groups and decoded slices against the oracle."""
    U.need_gpu()
    cfg = synth.CONFIGS["34b"]
    lvd = cfg.levels[0]
    X16 = synth.generate(cfg)
    x = U.to_dev(X16).to(torch.bfloat16)
    del X16
    Xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
    print("generated 34b bf16", flush=True)
    Tc = cfg.tokens // 4
    shp = C.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens, C.CG_DTYPE_BF16)
    cshp = C.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, Tc, cfg.chunk_tokens, C.CG_DTYPE_BF16)
    lv = U.codec.level_of(lvd)
    cd = U.codec.Codec(shp)
    tables = U.codec.Codec(cshp).build_tables(x[:, :, :, :Tc, :].contiguous(), lv, flags=C.CG_TABLES_ROBUST)
    out, offs = cd.encode(x, lv, tables)
    assert cd.read_status() == 0
    refs, n = cd.refs_for(out, offs)
    y = cd.decode([lv], [tables], refs, n)
    assert cd.read_status() == 0
    rng = np.random.default_rng(3)
    blob = U.u8(tables[:cd.format_bytes(lv)])
    G = len(lvd.steps)
    # tables: robust normalisation of the calibration counts
    Xc = np.ascontiguousarray(Xb[:, :, :, :Tc, :])
    ocshp = U.O.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, Tc, cfg.chunk_tokens, U.O.BF16)
    f = U.O.table_f(blob, ocshp, G)
    for _ in range(4):
        g, kv, h, d = int(rng.integers(G)), int(rng.integers(2)), int(rng.integers(cfg.kv_heads)), \
            int(rng.integers(cfg.head_dim))
        counts, _ = U.O.table_counts(ocshp, lvd.layer_group, lvd.steps, Xc, g, kv, h, d)
        assert np.array_equal(f[g, kv, h, d], U.O.normalize(counts, robust=True)), (g, kv, h, d)
    del Xc
    # groups of the whole tensor coded with the calibration tables
    oshp = U.O.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens, U.O.BF16)
    o = offs.cpu().numpy()
    S = cfg.head_dim // 64
    gpc = cfg.layers * 2 * cfg.kv_heads * S
    for c in [cfg.n_chunks - 1] + [int(rng.integers(cfg.n_chunks)) for _ in range(3)]:
        l, kv, h, j = (int(rng.integers(cfg.layers)), int(rng.integers(2)), int(rng.integers(cfg.kv_heads)),
                       int(rng.integers(S)))
        w = U.O.encode_group(oshp, blob, Xb, c, l, kv, h, j)
        rec = U.u8(out[int(o[c]):int(o[c + 1])])
        got = F.record_group(rec, gpc, ((l * 2 + kv) * cfg.kv_heads + h) * S + j)
        assert np.array_equal(got, w), (c, l, kv, h, j)
    # decoded slices
    for _ in range(3):
        l, kv, h = int(rng.integers(cfg.layers)), int(rng.integers(2)), int(rng.integers(cfg.kv_heads))
        st = lvd.steps[lvd.layer_group[l]]
        ref = F.npref.dequantize_bits(F.npref.quantize_bits(Xb[l, kv, h], st, 1), st, 1)
        assert np.array_equal(y[l, kv, h].cpu().view(torch.int16).numpy().view(np.uint16), ref), (l, kv, h)
    print("34b bf16 robust ratio %.3f:1" % (2 * Xb.size / int(o[-1])), flush=True)
