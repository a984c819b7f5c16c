"""Seeded synthetic KV tensors and the five workload configurations.

This module only draws inputs. It holds none of the codec's arithmetic, so
both the HIP path and the CPU oracle can use it without sharing code.

The pages measure on real prompts (legal, medical and financial documents,
dialogue) that are not available here. The generator stands in for them with
the statistical structure the method relies on:

* neighbouring tokens are similar ("CacheGen实战", section 1: adjacent tokens
  behave like consecutive video frames) -> a stationary AR(1) process along
  the token axis;
* channels differ in spread ("CacheGen：...技术解析", section on channel-aware
  quantization) -> a lognormal per-channel scale, 1 % outlier channels at 10x;
* deeper layers are coarser (section 1 of "CacheGen实战") -> scale grows with
  the layer index.

Recipe (per layer, seeded by [0, config_id, layer]):
    scale[kv,h,d] = exp(0.5*N(0,1)) * (1 + layer/4) * (10 if U(0,1) < 0.01 else 1)
    e[kv,h,t,d]   = N(0,1)  or  standard_t(3)/sqrt(3)
    z_0 = e_0 ;  z_t = rho*z_{t-1} + sqrt(1-rho^2)*e_t
    X = fp16(clip(scale*z, -65504, 65504))      layout [layer][K|V][head][token][dim]
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

FP16_MAX = 65504.0


@dataclasses.dataclass(frozen=True)
class Level:
    name: str
    level_id: int
    steps: tuple          # quantization step per layer group
    layer_group: tuple    # layer -> group index


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    config_id: int
    layers: int
    kv_heads: int
    head_dim: int
    tokens: int
    rho: float
    innovations: str      # "normal" or "t3"
    chunk_tokens: int
    levels: tuple         # one or more Level
    paged: bool = False
    block_tokens: int = 16

    @property
    def n_elements(self) -> int:
        return self.layers * 2 * self.kv_heads * self.tokens * self.head_dim

    @property
    def fp16_bytes(self) -> int:
        return 2 * self.n_elements

    @property
    def n_chunks(self) -> int:
        return -(-self.tokens // self.chunk_tokens)


def _ranges(bounds, layers):
    """Layer -> group map from inclusive [lo, hi] ranges."""
    lg = [None] * layers
    for g, (lo, hi) in enumerate(bounds):
        for layer in range(lo, hi + 1):
            lg[layer] = g
    assert all(v is not None for v in lg)
    return tuple(lg)


# Step presets of "CacheGen实战", section 3.1 (high / balanced / fast).
PRESET_STEPS = {
    "high": (0.3, 0.8, 1.2),
    "balanced": (0.5, 1.0, 1.5),
    "fast": (0.8, 1.5, 2.0),
}
LEVEL_IDS = {"high": 0, "balanced": 1, "fast": 2}

_LG_7B = _ranges([(0, 10), (11, 21), (22, 31)], 32)
_LG_34B = _ranges([(0, 15), (16, 31), (32, 47)], 48)


def _level(name, lg):
    return Level(name, LEVEL_IDS[name], PRESET_STEPS[name], lg)


CONFIGS = {
    "tiny": Config("tiny", 1, 4, 2, 64, 1024, 0.95, "normal", 256,
                   (Level("balanced", 1, (0.5, 1.0, 1.5), (0, 1, 1, 2)),)),
    "7b": Config("7b", 2, 32, 32, 128, 8192, 0.95, "normal", 1536,
                 (_level("balanced", _LG_7B),)),
    "34b": Config("34b", 3, 48, 8, 128, 32768, 0.97, "normal", 1536,
                  (_level("high", _LG_34B),)),
    "long": Config("long", 4, 48, 8, 128, 81920, 0.97, "normal", 1536,
                   (_level("high", _LG_34B), _level("balanced", _LG_34B),
                    _level("fast", _LG_34B))),
    "stream": Config("stream", 5, 32, 32, 128, 16384, 0.95, "t3", 1536,
                     (_level("balanced", _LG_7B),), paged=True),
}


def generate_layer(cfg: Config, layer: int, tokens: int | None = None) -> np.ndarray:
    """fp16 array [2][H][T][D] for one layer (T may be cut to `tokens`)."""
    from scipy.signal import lfilter

    T = cfg.tokens if tokens is None else tokens
    H, D = cfg.kv_heads, cfg.head_dim
    rng = np.random.default_rng([0, cfg.config_id, layer])
    scale = np.exp(0.5 * rng.standard_normal((2, H, D)))
    scale *= 1.0 + layer / 4.0
    scale *= np.where(rng.random((2, H, D)) < 0.01, 10.0, 1.0)
    if cfg.innovations == "normal":
        e = rng.standard_normal((2, H, cfg.tokens, D))
    else:
        e = rng.standard_t(3, size=(2, H, cfg.tokens, D)) / np.sqrt(3.0)
    e = e[:, :, :T, :]
    c = np.sqrt(1.0 - cfg.rho * cfg.rho)
    # z_t = rho*z_{t-1} + c*e_t with z_0 = e_0: feed e_0/c as the first input.
    e[:, :, 0, :] /= c
    z = lfilter([c], [1.0, -cfg.rho], e, axis=2)
    x = np.clip(z * scale[:, :, None, :], -FP16_MAX, FP16_MAX)
    return x.astype(np.float16)


def _gen_into(args):
    cfg, layer, T, path, offset = args
    arr = generate_layer(cfg, layer, T)
    mm = np.memmap(path, dtype=np.float16, mode="r+", offset=offset, shape=arr.shape)
    mm[...] = arr
    mm.flush()
    return layer


def generate(cfg: Config, tokens: int | None = None, workers: int | None = None) -> np.ndarray:
    """fp16 array [L][2][H][T][D]. Layers are independent draws, so they are
    generated in parallel processes; the result does not depend on `workers`."""
    T = cfg.tokens if tokens is None else tokens
    shape = (cfg.layers, 2, cfg.kv_heads, T, cfg.head_dim)
    per_layer = 2 * cfg.kv_heads * T * cfg.head_dim
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if workers <= 1 or cfg.layers == 1 or per_layer * cfg.layers < (1 << 22):
        out = np.empty(shape, dtype=np.float16)
        for layer in range(cfg.layers):
            out[layer] = generate_layer(cfg, layer, T)
        return out
    import tempfile
    fd, path = tempfile.mkstemp(prefix="cgkv_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    os.close(fd)
    try:
        total = per_layer * cfg.layers * 2
        with open(path, "wb") as f:
            f.truncate(total)
        jobs = [(cfg, layer, T, path, layer * per_layer * 2) for layer in range(cfg.layers)]
        with ProcessPoolExecutor(max_workers=workers) as ex:
            list(ex.map(_gen_into, jobs))
        mm = np.memmap(path, dtype=np.float16, mode="r", shape=shape)
        out = np.array(mm)
        del mm
    finally:
        os.unlink(path)
    return out


def level_mix(cfg: Config) -> np.ndarray:
    """Per-chunk level index for the multi-level decode (seeded)."""
    return np.random.default_rng([0, cfg.config_id, 999]).integers(0, len(cfg.levels), cfg.n_chunks)


def block_table(cfg: Config) -> np.ndarray:
    """Seeded random permutation of the 16-token blocks (int32)."""
    nb = -(-cfg.tokens // cfg.block_tokens)
    return np.random.default_rng([0, cfg.config_id, 999]).permutation(nb).astype(np.int32)


def random_kv(L, H, D, T, seed, scale=3.0, rho=0.9, dtype=np.float16):
    """Small generic AR(1) tensor for tests of arbitrary shapes."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(seed)
    e = rng.standard_normal((L, 2, H, T, D))
    c = np.sqrt(1 - rho * rho)
    e[:, :, :, 0, :] /= c
    z = lfilter([c], [1.0, -rho], e, axis=3)
    s = np.exp(0.5 * rng.standard_normal((L, 2, H, 1, D))) * scale
    return np.clip(z * s, -FP16_MAX, FP16_MAX).astype(dtype)


BF16_MAX = 3.3895313892515355e38


def random_kv_bf16(L, H, D, T, seed, scale=3.0, rho=0.9):
    """As random_kv, as raw bfloat16 bits (uint16): the same AR(1) draw,
    rounded to nearest-even bfloat16 by torch. A large `scale` exercises the
    range bfloat16 has beyond fp16."""
    import torch
    from scipy.signal import lfilter
    rng = np.random.default_rng(seed)
    e = rng.standard_normal((L, 2, H, T, D))
    c = np.sqrt(1 - rho * rho)
    e[:, :, :, 0, :] /= c
    z = lfilter([c], [1.0, -rho], e, axis=3)
    s = np.exp(0.5 * rng.standard_normal((L, 2, H, 1, D))) * scale
    x = np.clip(z * s, -BF16_MAX, BF16_MAX).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bandwidth_trace(n: int, seed: int = 0) -> np.ndarray:
    """Seeded synthetic link bandwidth in Gbit/s, one value per chunk: a
    random walk in log space between 0.05 and 20 Gbit/s (the pages' links range
    from 100 Mbit/s to 10 Gbit/s), so every level of the bandwidth policy is
    visited."""
    rng = np.random.default_rng([0, 77, seed])
    steps = rng.normal(0.0, 0.6, n)
    logb = np.log(3.0) + np.cumsum(steps)
    return np.exp(np.clip(logb, np.log(0.05), np.log(20.0)))
