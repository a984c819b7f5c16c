"""The whole-tensor checks of the full-size GPU tests, run on the CPU with
the oracle's own outputs on the tiny workload: the tables built slice by
slice ((layer group, head) sub-tensors) equal the whole tensor's, records
compare byte for byte, and the oracle's decode equals numpy's
dequant(quant(x)) everywhere. A planted difference is found."""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth
from oracle import oracle as O
from tests import fullsize as F


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    lvd = cfg.levels[0]
    X = synth.generate(cfg)
    oshp = O.shape_of(cfg)
    blob, _ = O.build_tables(oshp, lvd.level_id, lvd.layer_group, lvd.steps, X)
    data, offs = O.encode_all(oshp, blob, X)
    Y = O.decode_all(oshp, blob, data, offs)
    return cfg, lvd, X, blob, data, offs, Y


def test_tables_by_slice_equal_whole_tensor_tables(tiny):
    cfg, lvd, X, blob, *_ = tiny
    assert F.check_all_tables(cfg, lvd, X, blob) == len(lvd.steps) * 2 * cfg.kv_heads * cfg.head_dim
    bad = blob.copy()
    f_off = O.tables_f_offset(O.shape_of(cfg), len(lvd.steps))
    bad[f_off + 2 * 300] ^= 1
    with pytest.raises(AssertionError):
        F.check_all_tables(cfg, lvd, X, bad)


def test_records_compare_every_byte(tiny):
    cfg, lvd, X, blob, data, offs, _ = tiny
    rec = lambda k: data[int(offs[k]):int(offs[k + 1])]  # noqa: E731
    assert F.check_all_records(cfg, X, blob, rec, list(range(cfg.n_chunks))) == len(data)
    planted = data.copy()
    planted[int(offs[2]) + 5000] ^= 0x10
    with pytest.raises(AssertionError):
        F.check_all_records(cfg, X, blob, lambda k: planted[int(offs[k]):int(offs[k + 1])],
                            list(range(cfg.n_chunks)))


def test_decoded_compare_every_element(tiny):
    cfg, lvd, X, _, _, _, Y = tiny
    steps = [lvd.steps[g] for g in lvd.layer_group]
    assert F.check_all_decoded(cfg, X, steps, lambda l: Y[l]) == X.size
    ts = [(slice(0, 500), steps), (slice(500, None), steps)]
    assert F.check_all_decoded(cfg, X, None, lambda l: Y[l], token_steps=ts) == X.size
    Y2 = Y.copy()
    Y2[3, 1, 0, 777, 5] ^= 1
    with pytest.raises(AssertionError):
        F.check_all_decoded(cfg, X, steps, lambda l: Y2[l])
