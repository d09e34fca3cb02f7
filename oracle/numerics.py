"""Elementary definitions used by the oracle, in float64.

Every function here is the textbook definition written out; none is blocked,
fused or reordered.  Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even.

    bfloat16 keeps 8 significant bits and the float32 exponent range; values
    below 2^-126 are subnormal with spacing 2^-133.  Returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # subnormal range keeps spacing 2^-133
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)   # np.rint: ties to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(dtype: str):
    """The storage rounding of a configuration's activations: bf16 or f32."""
    if dtype == "bf16":
        return round_bf16
    if dtype == "f32":
        return round_f32
    raise ValueError(dtype)


def matmul_nt(x: np.ndarray, W: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """x @ W^T in float64 for W stored [out, in] (any float dtype).

    W is widened to float64 a block of rows at a time only to bound memory;
    every output element is still one float64 dot product over the full
    input dimension.
    """
    x = np.asarray(x, dtype=np.float64)
    n_out = W.shape[0]
    out = np.empty(x.shape[:-1] + (n_out,), dtype=np.float64)
    for r0 in range(0, n_out, chunk):
        blk = np.asarray(W[r0:r0 + chunk], dtype=np.float64)
        out[..., r0:r0 + chunk] = x @ blk.T
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def logsumexp(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    return np.squeeze(m, axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def rope_angles(positions: np.ndarray, d: int, base: float) -> np.ndarray:
    """Angles pos * base^(-2i/d) for i < d/2, shape [n_pos, d/2] (float64)."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding, rotate-half form, on the last axis of x [n_pos, ..., d].

    Dimension i is paired with i + d/2 and the pair is rotated by the angle
    pos * base^(-2i/d).
    """
    d = x.shape[-1]
    ang = rope_angles(positions, d, base)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    x1 = x[..., : d // 2]
    x2 = x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v with no mask: q [n_q, d], keys/vals [n_k, d]."""
    d = q.shape[-1]
    s = (q @ keys.T) / np.sqrt(d)
    return softmax(s, axis=-1) @ vals


def top2_gap(x: np.ndarray) -> np.ndarray:
    """Largest minus second-largest value along the last axis."""
    if x.shape[-1] < 2:
        return np.full(x.shape[:-1], np.inf)
    part = np.partition(x, -2, axis=-1)
    return part[..., -1] - part[..., -2]


def argmax_first(x: np.ndarray) -> np.ndarray:
    """Index of the maximum along the last axis, lowest index among equal maxima."""
    return np.argmax(x, axis=-1)
