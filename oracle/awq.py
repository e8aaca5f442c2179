"""AWQ W4A16 GEMV for the adaLN / modulation projections (oracle; test infrastructure).

The pages only say these precision-sensitive, low-compute projections keep
16-bit activations and 4-bit weights (donmalab.com page, section on the two
schemes; remio.ai page, section on the loading path). The arithmetic below is
the textbook asymmetric min/max group quantiser with an activation-aware
per-input-channel scale s_c folded into the weight:

  W'[k, n] = W[k, n] / inv_s[k] with inv_s = fp32(1 / s_c) (fp64, rounded to fp32)
  per (n, group g of 64 input channels):
     mn, mx = min, max of W'[k in g, n]
     s  = fp16(max(mx - mn, 1e-5) / 15)          (fp32 arithmetic, RTNE)
     z  = clamp(rtne(-mn * fp32(1 / s)), 0, 15)  (stored as an fp16 integer)
     q  = clamp(rtne(W' * fp32(1 / s)) + z, 0, 15)
  Y[m, n] = sum_k (fp32(x[m, k]) * inv_s[k]) (q - z) s + bias[n]   (fp64)

Codes are unsigned nibbles, stored [N][K/2] with element 2i in the low nibble
of byte i; scale and zero are fp16 [N][K/64]. The GEMV reads the codes in a
tile layout, [N/16][K/128][16][64 bytes] (``tile_for_gemv``): block (t, j, c)
is bytes 64j .. 64j + 63 of the plain row of column 16t + c; and the scales
and zero points as [N/16][K/64][16] (``tile_scales_for_gemv``). Both are
permutations and change no value.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numfmt import bf16_bits_to_f32, f32_to_f16, f64_to_bf16_bits

GROUP = 64


@dataclass
class AwqWeights:
    K: int
    N: int
    inv_s: np.ndarray        # fp32 [K]
    codes: np.ndarray        # uint8 [N, K] in 0..15
    qw: np.ndarray           # packed u8 [N, K/2]
    scale: np.ndarray        # fp16 [N, K/64]
    zero: np.ndarray         # fp16 [N, K/64] (integers 0..15)
    bias: np.ndarray | None  # bf16 bits [N]
    qwt: np.ndarray | None = None      # packed codes in the GEMV tile layout (K % 128 == 0)
    scale_t: np.ndarray | None = None  # scale in the GEMV tile layout [N/16][K/64][16]
    zero_t: np.ndarray | None = None   # zero point in the GEMV tile layout


def qasym64(v: np.ndarray):
    """Asymmetric 4-bit quantisation of groups along the last axis (float32
    [..., 64]) -> (scale fp16, zero fp16, codes uint8)."""
    v = np.asarray(v, np.float32)
    mn = v.min(axis=-1)
    mx = v.max(axis=-1)
    rng = np.maximum((mx - mn).astype(np.float32), np.float32(1e-5))
    s16 = f32_to_f16((rng / np.float32(15.0)).astype(np.float32))
    sf = s16.astype(np.float32)
    inv = (np.float32(1.0) / sf).astype(np.float32)
    z = np.clip(np.rint((-mn * inv).astype(np.float32)), 0, 15)
    q = np.clip(np.rint((v * inv[..., None]).astype(np.float32)) + z[..., None], 0, 15)
    return s16, z.astype(np.float16), q.astype(np.uint8)


def pack_u4(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    if c.max(initial=0) > 15:
        raise ValueError("codes out of [0, 15]")
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_u4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def tile_for_gemv(packed: np.ndarray) -> np.ndarray:
    """Plain packed rows [N][K/2] -> the tile layout [N/16][K/128][16][64] as a
    flat byte array: block (t, j, c) = packed[16 t + c, 64 j : 64 j + 64]."""
    p = np.asarray(packed, np.uint8)
    N, half_k = p.shape
    if N % 16 or half_k % 64:
        raise ValueError("tile layout needs N % 16 == 0 and K % 128 == 0")
    out = np.empty(N * half_k, np.uint8)
    pos = 0
    for t in range(N // 16):
        for j in range(half_k // 64):
            for c in range(16):
                out[pos:pos + 64] = p[16 * t + c, 64 * j:64 * j + 64]
                pos += 64
    return out


def tile_scales_for_gemv(a: np.ndarray) -> np.ndarray:
    """Per-(column, group) values [N][G] -> the tile layout [N/16][G][16] as a
    flat array: entry (t, g, c) = a[16 t + c, g]."""
    a = np.asarray(a)
    N, G = a.shape
    if N % 16:
        raise ValueError("tile layout needs N % 16 == 0")
    out = np.empty(N * G, a.dtype)
    pos = 0
    for t in range(N // 16):
        for g in range(G):
            for c in range(16):
                out[pos] = a[16 * t + c, g]
                pos += 1
    return out


def prepare_awq(w_bits: np.ndarray, chan_scale, bias_bits=None) -> AwqWeights:
    w = bf16_bits_to_f32(w_bits)
    K, N = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    sc = np.ones(K, np.float64) if chan_scale is None else np.asarray(chan_scale, np.float64)
    inv_s = (1.0 / sc).astype(np.float32)
    wp = (w.astype(np.float64) / inv_s.astype(np.float64)[:, None]).astype(np.float32)
    groups = np.ascontiguousarray(wp.T).reshape(N, K // GROUP, GROUP)
    s, z, q = qasym64(groups)
    codes = q.reshape(N, K)
    packed = pack_u4(codes)
    tiled = N % 16 == 0 and K % 128 == 0
    return AwqWeights(K, N, inv_s, codes, packed, s, z,
                      None if bias_bits is None else np.asarray(bias_bits, np.uint16),
                      tile_for_gemv(packed) if tiled else None,
                      tile_scales_for_gemv(s) if tiled else None,
                      tile_scales_for_gemv(z) if tiled else None)


def gemv(x_bits: np.ndarray, wts: AwqWeights) -> np.ndarray:
    """Y64 [M, N] = (fp32(x) * inv_s) @ dequant(W) + bias, in fp64."""
    x = bf16_bits_to_f32(x_bits)
    xs = (x * wts.inv_s[None, :]).astype(np.float32).astype(np.float64)
    q = wts.codes.astype(np.float64).reshape(wts.N, wts.K // GROUP, GROUP)
    deq = (q - wts.zero.astype(np.float64)[..., None]) * wts.scale.astype(np.float64)[..., None]
    y = xs @ deq.reshape(wts.N, wts.K).T
    if wts.bias is not None:
        y += bf16_bits_to_f32(wts.bias).astype(np.float64)[None, :]
    return y


def output_bf16(y64):
    return f64_to_bf16_bits(y64)
