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
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    C.cg_stream_decode_paged(cd.shp, [lv], [tables], host, o.astype(np.uint64), None, n, staging, refs2,
                             pool2, NB, torch.from_numpy(bt).cuda(), cd.status, copy_stream=copy_stream)
    e1.record()
    assert cd.read_status() == 0
    ms = e0.elapsed_time(e1)
    print("streamed %d records, %.1f MB in %.2f ms (%.1f GB/s host-to-device incl. decode)" % (
        n, o[-1] / 1e6, ms, o[-1] / ms / 1e6), flush=True)
    assert torch.equal(pool2.view(torch.int16), pool.view(torch.int16))
