"""Rounding and element-wise textbook functions used by the oracle (float64 math).

Storage contract for bf16 models: what is stored in bf16 is the weights and
the KV cache -- each column's k (after the positional rotation) and v are
rounded to bf16 (round to nearest, ties to even) because that is the form the
cache keeps them in.  Every activation (residual stream, RMSNorm outputs, q,
attention output, SwiGLU product, gated-delta-rule quantities, logits) is a
float32 value: one rounding of the float64 result.
"""
import numpy as np


def f32(x) -> np.ndarray:
    """Round (float64) values to float32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16(x) -> np.ndarray:
    """Round to float32, then to bf16 with round-to-nearest-even; returned as float32.

    Written on the bit pattern: add 0x7FFF plus the lowest kept bit, drop the
    low 16 bits.  NaN stays NaN.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def store(x, dtype: str) -> np.ndarray:
    """Round a float64 value to the storage precision of a model ("bf16" or "f32")."""
    return bf16(x) if dtype == "bf16" else f32(x)


def rmsnorm(x, gain, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, along the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding over the full head dimension.

    x: [..., n_heads, d]; pos: [...] absolute positions (broadcast over heads).
    Pair (i, i + d/2) is rotated by angle pos * theta^(-2i/d).  theta == 0 means
    no positional encoding.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta == 0.0:
        return x
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv_freq   # [..., 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)
