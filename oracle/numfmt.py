"""Rounding to the storage formats the layer uses (oracle; test infrastructure).

* bf16: 1 sign, 8 exponent, 7 mantissa bits. Round to nearest, ties to even,
  subnormals kept, NaN quietened. Written bit by bit from the IEEE-754 rule.
* fp16: IEEE binary16; numpy's float32 -> float16 cast is the IEEE RTNE
  conversion (subnormals kept) and serves as the library primitive.

The pages only say the low-rank branch is 16-bit and the pipelines run BF16
(remio.ai page, "memory alone is not enough" section); the rounding mode
(RTNE everywhere) is the reading taken for the open point.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.uint32(0x7F7F0000).view(np.float32))


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    isnan = (b & 0x7FFFFFFF) > 0x7F800000
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    qnan = ((b >> 16) | 0x0040) & 0xFFFF
    return np.where(isnan, qnan, r).astype(np.uint16)


def f64_to_bf16_bits(y) -> np.ndarray:
    """float64 -> bf16 bit pattern with a single round to nearest even.

    The value is split as m * 2**e (frexp, m in [0.5, 1)); bf16 keeps 8
    significant bits, so the quantum is 2**(e - 8), but never finer than the
    smallest bf16 subnormal 2**-133. Magnitudes that round above the largest
    finite bf16 become infinity."""
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.uint16)
    nan = np.isnan(y)
    _, e = np.frexp(y)
    qexp = np.maximum(e - 8, -133)
    scaled = np.ldexp(y, -qexp)          # exact: power-of-two scaling
    r = np.rint(scaled)                  # RTNE
    val = np.ldexp(r, qexp)              # exactly representable in bf16 (or overflow)
    big = np.abs(val) > BF16_MAX
    val = np.where(big, np.copysign(np.inf, y), val)
    with np.errstate(over="ignore"):
        f = val.astype(np.float32)       # exact for every bf16 value
    out[...] = (f.view(np.uint32) >> 16).astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def f32_to_f16(x) -> np.ndarray:
    """float32 -> float16 (IEEE round to nearest even, subnormals kept)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def f16_bits(h) -> np.ndarray:
    return np.asarray(h, dtype=np.float16).view(np.uint16)


def f16_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16)
