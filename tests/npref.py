"""Independent numpy routes used to pin the oracle (no oracle code here).

Quantization goes through binary64 and rounds once to binary32: for a
binary32 quotient that double rounding is innocuous (53 >= 2*24 + 2), so this
equals the IEEE binary32 divide the definition asks for.
"""
import numpy as np


def quantize(x16: np.ndarray, step: float) -> np.ndarray:
    xf = x16.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        v = (xf / np.float64(np.float32(step))).astype(np.float32)
        r = np.rint(v)
        r = np.nan_to_num(r, nan=0.0, posinf=1e9, neginf=-1e9)
    return np.clip(r, -32768, 32767).astype(np.int64)


def dequantize(q: np.ndarray, step: float) -> np.ndarray:
    with np.errstate(over="ignore"):
        return (q.astype(np.float32) * np.float32(step)).astype(np.float16)


def quantize_tensor(X, layer_group, steps):
    """int64 q with the layout of X [L][2][H][T][D]."""
    return np.stack([quantize(X[l], steps[layer_group[l]]) for l in range(X.shape[0])])


def reconstruct(X, layer_group, steps):
    q = quantize_tensor(X, layer_group, steps)
    return np.stack([dequantize(q[l], steps[layer_group[l]]) for l in range(X.shape[0])])


def symbols(q, chunk):
    """Per-chunk token deltas (wrap 2^16) -> symbols; list of arrays [L][2][H][n-1][D]."""
    T = q.shape[3]
    out = []
    for t0 in range(0, T, chunk):
        qc = q[:, :, :, t0:min(t0 + chunk, T), :]
        d = np.diff(qc, axis=3)
        d = (d + 32768) % 65536 - 32768
        out.append(np.where(np.abs(d) <= 127, d + 127, 255))
    return out


def counts(X, layer_group, steps, chunk, n_groups):
    """u64 counts [G][2][H][D][256] by numpy bincount."""
    L, _, H, T, D = X.shape
    q = quantize_tensor(X, layer_group, steps)
    cnt = np.zeros((n_groups, 2, H, D, 256), dtype=np.uint64)
    for sym in symbols(q, chunk):
        for l in range(L):
            s = sym[l]  # [2][H][n-1][D]
            idx = ((np.arange(2)[:, None, None, None] * H + np.arange(H)[None, :, None, None]) * D
                   + np.arange(D)[None, None, None, :]) * 256 + s
            cnt[layer_group[l]] += np.bincount(idx.ravel(), minlength=2 * H * D * 256).reshape(
                2, H, D, 256).astype(np.uint64)
    return cnt


# ---- bfloat16 routes (torch's CPU conversions are the library routine) ----
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b.copy()).view(torch.bfloat16).to(torch.float64).numpy()


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def quantize_bits(x_bits: np.ndarray, step: float, dtype: int) -> np.ndarray:
    """quantize() for raw 16-bit element bits of either type (0 fp16, 1 bf16)."""
    if dtype == 0:
        return quantize(np.ascontiguousarray(x_bits, dtype=np.uint16).view(np.float16), step)
    xf = bf16_to_f64(x_bits)
    with np.errstate(invalid="ignore", over="ignore"):
        v = (xf / np.float64(np.float32(step))).astype(np.float32)
        r = np.rint(v)
        r = np.nan_to_num(r, nan=0.0, posinf=1e9, neginf=-1e9)
    return np.clip(r, -32768, 32767).astype(np.int64)


def dequantize_bits(q: np.ndarray, step: float, dtype: int) -> np.ndarray:
    if dtype == 0:
        return dequantize(q, step).view(np.uint16)
    with np.errstate(over="ignore"):
        return f32_to_bf16_bits(q.astype(np.float32) * np.float32(step))


def reconstruct_bits(X_bits, layer_group, steps, dtype):
    return np.stack([dequantize_bits(quantize_bits(X_bits[l], steps[layer_group[l]], dtype),
                                     steps[layer_group[l]], dtype) for l in range(X_bits.shape[0])])


def counts_bits(X_bits, layer_group, steps, chunk, n_groups, dtype):
    """counts() for raw element bits of either type."""
    L, _, H, T, D = X_bits.shape
    q = np.stack([quantize_bits(X_bits[l], steps[layer_group[l]], dtype) for l in range(L)])
    cnt = np.zeros((n_groups, 2, H, D, 256), dtype=np.uint64)
    for sym in symbols(q, chunk):
        for l in range(L):
            s = sym[l]
            idx = ((np.arange(2)[:, None, None, None] * H + np.arange(H)[None, :, None, None]) * D
                   + np.arange(D)[None, None, None, :]) * 256 + s
            cnt[layer_group[l]] += np.bincount(idx.ravel(), minlength=2 * H * D * 256).reshape(
                2, H, D, 256).astype(np.uint64)
    return cnt
