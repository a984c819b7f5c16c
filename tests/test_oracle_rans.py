"""rANS group coder pins: hand-derived streams, a closed form for
power-of-two tables, brute force on tiny alphabets and information bounds.

Definition under test ("CacheGen实战" section 1, grouped entropy coding of
token deltas; 12-bit static rANS reading): per lane a 32-bit state in
[2^16, 2^32), renormalised with 16-bit words, lanes interleaved word by word.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rans_examples.json")


def table_from(d):
    f = np.zeros(256, dtype=np.uint16)
    for k, v in d.items():
        f[int(k)] = v
    assert f.sum() == 4096
    return f


def symbols_of(q):
    """Symbols and escape payloads of one lane (numpy route, int64)."""
    d = np.diff(np.asarray(q, dtype=np.int64))
    d = (d + 32768) % 65536 - 32768
    sym = np.where(np.abs(d) <= 127, d + 127, 255)
    return sym, d


def tables_for(q):
    """Self-calibrated per-lane tables for q[64][n] (numpy counts -> oracle normalise)."""
    f = np.zeros((64, 256), dtype=np.uint16)
    for k in range(64):
        sym, _ = symbols_of(q[k])
        f[k] = O.normalize(np.bincount(sym, minlength=256).astype(np.uint64))
    return f


def expand(runs):
    return np.concatenate([np.full(r, v, dtype=np.uint16) for v, r in runs])


def test_hand_derived_examples():
    ex = json.load(open(GOLDEN))["examples"]
    for e in ex:
        q = np.tile(np.array(e["q"], dtype=np.int32), (64, 1))
        f = np.tile(table_from(e["f"]), (64, 1))
        words = O.encode_group_q(q, f)
        assert np.array_equal(words, expand(e["words"])), e["name"]
        rc, back = O.decode_group_q(words, q.shape[1], f)
        assert rc == O.OK and np.array_equal(back, q), e["name"]


def lane_example(e):
    q = np.array([ln["q"] for ln in e["lanes"]], dtype=np.int32)
    f = np.stack([table_from(ln["f"]) for ln in e["lanes"]])
    return q, f, np.array(e["words"], dtype=np.uint16)


def test_hand_derived_lane_examples():
    """Different data on every lane: within one token the renorm words come
    before the escape payloads, each block in ascending lane order, and a
    token's words come before the next token's (hand-derived streams)."""
    for e in json.load(open(GOLDEN))["lane_examples"]:
        q, f, want = lane_example(e)
        assert len(e["lanes"]) == 64 and q.shape == (64, 3)
        words = O.encode_group_q(q, f)
        assert np.array_equal(words, want), e["name"]
        rc, back = O.decode_group_q(want, 3, f)
        assert rc == O.OK and np.array_equal(back, q), e["name"]


def test_lane_examples_tell_orders_apart():
    """The goldens are not blind to the orders they pin: the stream with the
    renorm and escape blocks swapped, or with either block in descending
    lane order, is a different stream, and the oracle decoder rejects it or
    decodes other values."""
    e = json.load(open(GOLDEN))["lane_examples"][0]
    q, f, want = lane_example(e)
    cls = np.arange(64) % 4
    n_r = int(np.isin(cls, (0, 2)).sum())
    n_e = int(np.isin(cls, (1, 2)).sum())
    head, ren, esc = want[:192], want[192:192 + n_r], want[192 + n_r:]
    assert len(esc) == n_e
    variants = [np.concatenate([head, esc, ren]), np.concatenate([head, ren[::-1], esc]),
                np.concatenate([head, ren, esc[::-1]])]
    for v in variants:
        assert not np.array_equal(v, want)
        rc, back = O.decode_group_q(v, 3, f)
        assert rc != O.OK or not np.array_equal(back, q)
    # token order: the second example's renorm words (token 1) precede its
    # escape payloads (token 2)
    e2 = json.load(open(GOLDEN))["lane_examples"][1]
    q2, f2, want2 = lane_example(e2)
    swapped = np.concatenate([want2[:192], want2[224:], want2[192:224]])
    rc, back = O.decode_group_q(swapped, 3, f2)
    assert rc != O.OK or not np.array_equal(back, q2)


def random_q(rng, n, spread, jumps=0.0):
    q = np.zeros((64, n), dtype=np.int64)
    q[:, 0] = rng.integers(-32768, 32768, size=64)
    w = spread * np.exp(rng.standard_normal(64))
    steps = np.rint(rng.laplace(0, 1, size=(64, n - 1)) * w[:, None]).astype(np.int64)
    if jumps:
        mask = rng.random((64, n - 1)) < jumps
        steps[mask] = rng.integers(-65536, 65536, size=mask.sum())
    q[:, 1:] = q[:, :1] + np.cumsum(steps, axis=1)
    return ((q + 32768) % 65536 - 32768).astype(np.int32)


@pytest.mark.parametrize("seed,n,spread,jumps", [
    (0, 2, 1.0, 0.0), (1, 3, 0.1, 0.0), (2, 100, 1.0, 0.0), (3, 257, 5.0, 0.01),
    (4, 1536, 0.7, 0.0), (5, 700, 40.0, 0.05), (6, 64, 300.0, 0.2), (7, 1, 1.0, 0.0)])
def test_round_trip(seed, n, spread, jumps):
    rng = np.random.default_rng(seed)
    q = random_q(rng, n, spread, jumps)
    f = tables_for(q)
    words = O.encode_group_q(q, f)
    rc, back = O.decode_group_q(words, n, f)
    assert rc == O.OK
    assert np.array_equal(back, q)
    # escape count equals the payload words in the stream (independent count)
    esc = sum(int((symbols_of(q[k])[0] == 255).sum()) for k in range(64))
    assert len(words) >= 192 + esc


def test_wraparound_deltas():
    q = np.zeros((64, 4), dtype=np.int32)
    q[:, 0] = 32767
    q[:, 1] = -32768        # wrap16(-65535) = +1 -> ordinary symbol 128
    q[:, 2] = 32767         # -1
    q[:, 3] = -128          # wrap16(-32895) = 32641 -> escape
    f = tables_for(q)
    sym, d = symbols_of(q[0])
    assert list(sym) == [128, 126, 255]
    words = O.encode_group_q(q, f)
    rc, back = O.decode_group_q(words, 4, f)
    assert rc == O.OK and np.array_equal(back, q)
    # the escape payload is the wrapped difference as an unsigned 16-bit word
    assert np.count_nonzero(words[192:] == (32641 & 0xFFFF)) == 64


def test_escape_boundaries():
    for delta, is_esc in [(127, False), (-127, False), (128, True), (-128, True)]:
        q = np.zeros((64, 2), dtype=np.int32)
        q[:, 1] = delta
        sym, _ = symbols_of(q[0])
        assert (sym[0] == 255) == is_esc
        f = tables_for(q)
        words = O.encode_group_q(q, f)
        assert len(words) == 192 + (64 if is_esc else 0)
        rc, back = O.decode_group_q(words, 2, f)
        assert rc == O.OK and np.array_equal(back, q)


def test_power_of_two_tables_closed_form():
    """With f = 2^m every coding step adds exactly 12-m bits to the state and
    a renorm removes 16, so renorm counts and final states follow from bit
    lengths alone."""
    rng = np.random.default_rng(11)
    n = 600
    f_one = np.zeros(256, dtype=np.uint16)
    # symbols 120..134 with power-of-two frequencies summing to 4096
    pw = {127: 2048, 126: 512, 128: 512, 125: 256, 129: 256, 124: 128, 130: 128,
          123: 64, 131: 64, 122: 32, 132: 32, 121: 16, 133: 16, 120: 8, 134: 8, 0: 4, 254: 4,
          1: 2, 253: 2, 2: 1, 252: 1, 3: 1, 251: 1}
    for k, v in pw.items():
        f_one[k] = v
    assert f_one.sum() == 4096
    f = np.tile(f_one, (64, 1))
    syms = np.array(sorted(pw))
    p = np.array([pw[s] for s in syms], dtype=np.float64) / 4096
    q = np.zeros((64, n), dtype=np.int64)
    q[:, 0] = rng.integers(-1000, 1000, size=64)
    draws = rng.choice(syms, size=(64, n - 1), p=p) - 127
    q[:, 1:] = q[:, :1] + np.cumsum(draws, axis=1)
    q = ((q + 32768) % 65536 - 32768).astype(np.int32)
    words = O.encode_group_q(q, f)
    total_renorm = 0
    final_bits = []
    for k in range(64):
        sym, _ = symbols_of(q[k])
        bl = 17
        for s in sym[::-1]:
            m = int(f_one[s]).bit_length() - 1
            if bl >= m + 21:
                total_renorm += 1
                bl -= 16
            bl += 12 - m
        final_bits.append(bl)
    assert len(words) == 192 + total_renorm
    states = (words[:64].astype(np.uint64) << 16) | words[64:128].astype(np.uint64)
    assert [int(x).bit_length() for x in states] == final_bits


def test_brute_force_tiny_alphabet():
    """Every sequence of 7 symbols over a 3-symbol table on lane 0 decodes
    back, and distinct sequences give distinct streams."""
    f0 = table_from({126: 1000, 127: 2000, 128: 1096})
    f = np.tile(table_from({127: 4096}), (64, 1))
    f[0] = f0
    seen = {}
    for seq in itertools.product((-1, 0, 1), repeat=7):
        q = np.zeros((64, 8), dtype=np.int32)
        q[0, 1:] = np.cumsum(seq)
        words = O.encode_group_q(q, f)
        rc, back = O.decode_group_q(words, 8, f)
        assert rc == O.OK and np.array_equal(back, q)
        key = words.tobytes()
        assert key not in seen
        seen[key] = seq
    assert len(seen) == 3 ** 7


@pytest.mark.parametrize("seed", range(6))
def test_information_bound(seed):
    """Per coding step the state grows by log2(M/f) within log2(17/16) and
    shrinks by 16 bits (+ < log2(16/15)) per renorm word, so
    |16 R + log2 x_final - 16 - sum log2(M/f)| <= 0.0931 (n-1 + R) per lane."""
    rng = np.random.default_rng(100 + seed)
    n = [50, 300, 1536][seed % 3]
    q = random_q(rng, n, [0.3, 3.0, 30.0][seed % 3], 0.0 if seed < 3 else 0.01)
    f = tables_for(q)
    words = O.encode_group_q(q, f)
    esc = 0
    ce = 0.0
    for k in range(64):
        sym, _ = symbols_of(q[k])
        esc += int((sym == 255).sum())
        ce += float(np.sum(np.log2(4096.0 / f[k][sym].astype(np.float64))))
    R = len(words) - 192 - esc
    states = (words[:64].astype(np.uint64) << 16) | words[64:128].astype(np.uint64)
    gain = 16 * R + sum(math.log2(int(x)) - 16 for x in states)
    assert abs(gain - ce) <= 0.0931 * (64 * (n - 1) + R) + 1e-6
    # measured overhead is small in practice
    if n == 1536:
        assert gain <= ce * 1.01 + 64 * 32


def test_corrupt_streams_detected_or_contained():
    rng = np.random.default_rng(5)
    q = random_q(rng, 200, 2.0)
    f = tables_for(q)
    words = O.encode_group_q(q, f)
    # truncated stream: reads past the end
    assert O.decode_group_q(words[:-1], 200, f)[0] == O.ERR_CORRUPT
    # extra word: not all words consumed
    assert O.decode_group_q(np.append(words, 0), 200, f)[0] == O.ERR_CORRUPT
    # damaged state word: final state check fails for this fixed case
    w2 = words.copy()
    w2[3] ^= 0x0100
    assert O.decode_group_q(w2, 200, f)[0] == O.ERR_CORRUPT
    # too short for the head
    assert O.decode_group_q(words[:100], 200, f)[0] == O.ERR_CORRUPT


def test_symbol_absent_from_table_is_an_error():
    q = np.zeros((64, 3), dtype=np.int32)
    q[:, 2] = 1
    f = np.tile(table_from({127: 4096}), (64, 1))
    with pytest.raises(RuntimeError):
        O.encode_group_q(q, f)
