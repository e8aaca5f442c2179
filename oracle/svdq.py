"""SVDQuant W4A4 linear layer, step by step (oracle; test infrastructure).

What the pages fix (remio.ai page, section "SVDQuant moves hard values out of
4-bit"; donmalab.com page, core-challenge section):
  1. activation outliers are moved into the weights (smoothing);
  2. a small 16-bit low-rank branch represents the hardest part of the weight;
  3. the residual runs with 4-bit weights and 4-bit activations;
  4. the two results are added.
The remio.ai page adds that the original engine fused the low-rank
down-projection into input quantisation and the up-projection into the 4-bit
matmul; that is a kernel design, not arithmetic, and the oracle does neither.

Readings taken where the pages are silent (all listed in the design notes):
  * smoothing lambda[k] = ax[k]**alpha / aw[k]**(1-alpha) (alpha = 0.5) with
    ax, aw the per-input-channel absolute maxima of the calibration
    activations and of the weight; X_hat = X diag(1/lambda), W_hat = diag(lambda) W;
  * low-rank branch = truncated SVD of W_hat, L1 = bf16(U_r S_r), L2 = bf16(V_r^T);
  * residual R = W_hat - L1 L2 (from the rounded factors), rounded to fp32;
  * 4-bit = symmetric integers in [-7, 7], one fp16 scale per 64 consecutive
    input channels (per token row for X, per output column for R), scale =
    fp16(absmax / 7), codes = clamp(rtne(v * fp32(1 / scale)), -7, 7);
  * Y = X_hat L1 L2 + sum_g sx sw P_g + bias, with P_g the exact integer dot
    product of the codes of group g, then optional GELU (tanh form).

Storage format of the 4-bit codes (format v2; shared with the library only as
a documented layout, not as code): rows are K-contiguous and every run of 16
consecutive codes of a row is one little-endian 64-bit word. The word is
defined through the 96-bit stream T that holds the 16 codes as FP6 E2M3
values q / 8 (OCP microscaling formats: sign bit 5, exponent bits 3-4,
mantissa bits 0-2 of each 6-bit field; a code's field sits at bits 6e..6e+5
of T, its exponent bits are zero). The word keeps T[0:32) in bits 0-31 and
T[64:96) in bits 32-63; the 32 bits of T[32:64) are stored in the exponent
positions of those two parts (each bit of T[32:64) at the same offset in
the low half when that offset is an exponent position of T[0:32), else in
the high half, where it is an exponent position of T[64:96)). So the
word is a bit permutation of 16 sign-magnitude codes and the three 32-bit
thirds of T come back with masks alone. Weights are stored transposed,
[N][K/2].

Storage format of the scales (format v3): fp16, "quad-major": the scales of
the groups 4q .. 4q+3 of a row are 8 consecutive bytes, and quad q of all rows
comes before quad q+1, i.e. an array [ceil(G/4)][rows][4]; groups past the
last one (G = K/64 not a multiple of 4) hold 0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import linalg
from .numfmt import (bf16_bits_to_f32, f16_bits, f16_from_bits, f32_to_bf16_bits,
                     f32_to_f16, f64_to_bf16_bits)

GROUP = 64
QMAX = 7
F16_MAX = 65504.0


# --------------------------------------------------------------------------
# offline: calibration, smoothing, low-rank branch, residual quantisation
# --------------------------------------------------------------------------

def calib_absmax(x_f32: np.ndarray, w_f32: np.ndarray):
    """Per input channel k: ax[k] = max over tokens |X[m,k]|, aw[k] = max over
    outputs |W[k,n]| (W is K x N)."""
    ax = np.max(np.abs(x_f32), axis=0).astype(np.float32)
    aw = np.max(np.abs(w_f32), axis=1).astype(np.float32)
    return ax, aw


def smoothing(ax, aw, alpha: float):
    """lambda = ax**alpha / aw**(1-alpha) in fp64 (1 where either maximum is 0).
    Returns (lambda fp64, inv_lambda fp32). The online path multiplies by
    inv_lambda; the weight is divided by that same stored fp32 number, so that
    X_hat W_hat equals X W exactly in real arithmetic."""
    ax = np.asarray(ax, np.float64)
    aw = np.asarray(aw, np.float64)
    ok = (ax > 0) & (aw > 0)
    lam = np.ones_like(ax)
    lam[ok] = ax[ok] ** alpha / aw[ok] ** (1.0 - alpha)
    inv_lam = (1.0 / lam).astype(np.float32)
    return lam, inv_lam


def smooth_weight(w_f32: np.ndarray, inv_lam: np.ndarray) -> np.ndarray:
    """W_hat[k, n] = W[k, n] / inv_lambda[k] (fp64)."""
    return np.asarray(w_f32, np.float64) / np.asarray(inv_lam, np.float64)[:, None]


def lowrank_factors(w_hat: np.ndarray, rank: int, seed: int = 0):
    """L1 = bf16(U_r diag(s_r)) [K, r], L2 = bf16(V_r^T) [r, N] as bf16 bits,
    plus the singular values used."""
    if rank == 0:
        K, N = w_hat.shape
        return np.zeros((K, 0), np.uint16), np.zeros((0, N), np.uint16), np.zeros(0)
    u, s, vt = linalg.truncated_svd(w_hat, rank, seed=seed)
    l1 = f64_to_bf16_bits(u * s[None, :])
    l2 = f64_to_bf16_bits(vt)
    return l1, l2, s


def residual(w_hat: np.ndarray, l1_bits: np.ndarray, l2_bits: np.ndarray) -> np.ndarray:
    """R = W_hat - L1 L2 with the rounded factors, in fp64, then rounded to fp32."""
    l1 = bf16_bits_to_f32(l1_bits).astype(np.float64)
    l2 = bf16_bits_to_f32(l2_bits).astype(np.float64)
    return (w_hat - l1 @ l2).astype(np.float32)


def qsym64(v: np.ndarray):
    """Symmetric INT4 quantisation of groups along the last axis.

    v: float32 [..., 64]. For each group: amax = max |v|;
    s = fp16(min(amax / 7, 65504)) computed as one fp32 division then RTNE to
    fp16; if s == 0 every code is 0; else inv = fp32(1 / fp32(s)) (one
    correctly rounded division) and q = clamp(rtne(v * inv), -7, 7) with the
    product in fp32. Returns (s as fp16 [...], q as int8 [..., 64])."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=-1)
    s32 = np.minimum(amax / np.float32(QMAX), np.float32(F16_MAX)).astype(np.float32)
    s16 = f32_to_f16(s32)
    sf = s16.astype(np.float32)
    nz = sf > 0
    inv = np.zeros_like(sf)
    inv[nz] = np.float32(1.0) / sf[nz]
    prod = (v * inv[..., None]).astype(np.float32)
    q = np.clip(np.rint(prod), -QMAX, QMAX).astype(np.int8)
    q[~nz] = 0
    return s16, q


def group_view(a: np.ndarray) -> np.ndarray:
    rows, K = a.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    return a.reshape(rows, K // GROUP, GROUP)


def quantize_rows(v_f32: np.ndarray):
    """Qsym64 on every row-group of a [rows, K] float32 matrix.
    Returns (codes int8 [rows, K], scales fp16 [rows, K/64])."""
    s, q = qsym64(group_view(v_f32))
    return q.reshape(v_f32.shape), s


def dequantize_rows(codes: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """codes * scale per group, fp64."""
    q = group_view(codes.astype(np.float64))
    return (q * np.asarray(scales_f16, np.float16).astype(np.float64)[..., None]).reshape(codes.shape)


def _e2m3_word_positions() -> np.ndarray:
    """Bit position in the 64-bit storage word of (code e, bit b) for e < 16,
    b = 0, 1, 2 (magnitude bits) and b = 3 (sign), following the format-v2
    definition above: the E2M3 field of code e sits at stream bits 6e..6e+5
    (mantissa 6e..6e+2, exponent 6e+3..6e+4, sign 6e+5)."""
    exp_pos = {6 * e + 3 for e in range(16)} | {6 * e + 4 for e in range(16)}
    lo_holes = {t for t in exp_pos if t < 32}                # exponent bits of T[0:32)
    hi_holes = {t - 64 for t in exp_pos if t >= 64}          # exponent bits of T[64:96)
    pos = np.empty((16, 4), np.int64)
    for e in range(16):
        for b, off in enumerate((0, 1, 2, 5)):
            t = 6 * e + off
            if t < 32:
                pos[e, b] = t
            elif t >= 64:
                pos[e, b] = t - 32
            else:
                u = t - 32
                if u in lo_holes:
                    pos[e, b] = u
                elif u in hi_holes:
                    pos[e, b] = 32 + u
                else:
                    raise AssertionError("stream bit has no storage position")
    return pos


_WORD_POS = _e2m3_word_positions()


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int8 codes in [-7, 7], [rows, K] (K % 16 == 0) -> bytes [rows, K/2] in
    format v2 (see the module docstring). Zero is stored with sign 0."""
    c = np.asarray(codes, np.int16)
    if c.min(initial=0) < -QMAX or c.max(initial=0) > QMAX:
        raise ValueError("codes out of [-7, 7]")
    rows, k = c.shape
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    c = c.reshape(rows, k // 16, 16)
    mag = np.abs(c).astype(np.uint64)
    sgn = (c < 0).astype(np.uint64)
    word = np.zeros((rows, k // 16), np.uint64)
    for e in range(16):
        for b in range(3):
            word |= ((mag[:, :, e] >> np.uint64(b)) & np.uint64(1)) << np.uint64(_WORD_POS[e, b])
        word |= sgn[:, :, e] << np.uint64(_WORD_POS[e, 3])
    return word.astype("<u8").view(np.uint8).reshape(rows, k // 2)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4 -> int8 codes [rows, 2 * bytes]."""
    p = np.ascontiguousarray(np.asarray(packed, np.uint8))
    rows, nb = p.shape
    if nb % 8:
        raise ValueError("row length must be a multiple of 8 bytes")
    word = p.view("<u8").astype(np.uint64)
    out = np.empty((rows, nb // 8, 16), np.int8)
    for e in range(16):
        mag = np.zeros(word.shape, np.int64)
        for b in range(3):
            mag |= (((word >> np.uint64(_WORD_POS[e, b])) & np.uint64(1)).astype(np.int64) << b)
        neg = ((word >> np.uint64(_WORD_POS[e, 3])) & np.uint64(1)).astype(bool)
        out[:, :, e] = np.where(neg, -mag, mag)
    return out.reshape(rows, nb * 2)


def pack_scales(scales: np.ndarray) -> np.ndarray:
    """fp16 scales [rows, G] -> the quad-major storage array
    [ceil(G/4), rows, 4] (format v3, see the module docstring)."""
    s = np.asarray(scales, np.float16)
    rows, G = s.shape
    G4 = (G + 3) // 4
    out = np.zeros((G4, rows, 4), np.float16)
    for g in range(G):
        out[g // 4, :, g % 4] = s[:, g]
    return out


def unpack_scales(packed: np.ndarray, G: int) -> np.ndarray:
    """Inverse of pack_scales -> fp16 [rows, G] (the padding is dropped)."""
    p = np.asarray(packed, np.float16)
    G4, rows, four = p.shape
    if four != 4 or G4 != (G + 3) // 4:
        raise ValueError("not a quad-major scale array for this G")
    out = np.empty((rows, G), np.float16)
    for g in range(G):
        out[:, g] = p[g // 4, :, g % 4]
    return out


def pack_l1_tiles(l1_bits: np.ndarray) -> np.ndarray:
    """L1 (bf16 bits [K, r], r a multiple of 16) -> the L1 tile layout
    (format v4) as a flat uint16 array: for each 64-channel group g, 16-rank
    tile t, 32-channel step s and lane l = 0..63, eight values
    L1[64 g + 16 (l // 16) + 8 s + j, 16 t + l % 16] for j = 0..7, in the
    order (g, t, s, l, j)."""
    l1 = np.asarray(l1_bits, np.uint16)
    K, r = l1.shape
    if K % 64 or r % 16:
        raise ValueError("K must be a multiple of 64 and r of 16")
    out = np.empty(K * r, np.uint16)
    pos = 0
    for g in range(K // 64):
        for t in range(r // 16):
            for st in range(2):
                for lane in range(64):
                    k0 = 64 * g + 16 * (lane // 16) + 8 * st
                    out[pos:pos + 8] = l1[k0:k0 + 8, 16 * t + lane % 16]
                    pos += 8
    return out


def unpack_l1_tiles(packed: np.ndarray, K: int, r: int) -> np.ndarray:
    """Inverse of pack_l1_tiles -> bf16 bits [K, r]."""
    p = np.asarray(packed, np.uint16).reshape(-1)
    if p.size != K * r:
        raise ValueError("size does not match K * r")
    out = np.empty((K, r), np.uint16)
    pos = 0
    for g in range(K // 64):
        for t in range(r // 16):
            for st in range(2):
                for lane in range(64):
                    k0 = 64 * g + 16 * (lane // 16) + 8 * st
                    out[k0:k0 + 8, 16 * t + lane % 16] = p[pos:pos + 8]
                    pos += 8
    return out


@dataclass
class SvdqWeights:
    """Offline artefacts of one SVDQ layer (what a quantised checkpoint holds)."""
    K: int
    N: int
    rank: int
    inv_lambda: np.ndarray   # fp32 [K]
    l1: np.ndarray           # bf16 bits [K, r]
    l2: np.ndarray           # bf16 bits [r, N]
    qw_codes: np.ndarray     # int8 [N, K]
    qw: np.ndarray           # packed u8 [N, K/2]
    sw: np.ndarray           # fp16 [N, K/64]
    bias: np.ndarray | None  # bf16 bits [N]
    sigma: np.ndarray        # singular values used (diagnostics)
    w_hat: np.ndarray | None = None  # fp64 [K, N] (diagnostics; dropped for big layers)


def prepare_svdq(x_bits: np.ndarray, w_bits: np.ndarray, bias_bits, rank: int,
                 alpha: float = 0.5, svd_seed: int = 0, smooth: bool = True,
                 keep_w_hat: bool = False) -> SvdqWeights:
    """Offline preparation: calibration on X (the calibration set), smoothing,
    low-rank factors, residual, INT4 g64 quantisation of the residual."""
    x = bf16_bits_to_f32(x_bits)
    w = bf16_bits_to_f32(w_bits)
    K, N = w.shape
    if smooth:
        ax, aw = calib_absmax(x, w)
        _, inv_lam = smoothing(ax, aw, alpha)
    else:
        inv_lam = np.ones(K, np.float32)
    w_hat = smooth_weight(w, inv_lam)
    l1, l2, sig = lowrank_factors(w_hat, rank, seed=svd_seed)
    r = residual(w_hat, l1, l2)                 # [K, N] fp32
    codes, sw = quantize_rows(np.ascontiguousarray(r.T))   # per output column n
    return SvdqWeights(K, N, rank, inv_lam, l1, l2, codes, pack_int4(codes), sw,
                       None if bias_bits is None else np.asarray(bias_bits, np.uint16),
                       sig, w_hat if keep_w_hat else None)


# --------------------------------------------------------------------------
# online: activation quantisation, group partials, output
# --------------------------------------------------------------------------

@dataclass
class QuantAct:
    x_hat: np.ndarray    # fp32 [M, K]
    codes: np.ndarray    # int8 [M, K]
    qx: np.ndarray       # packed u8 [M, K/2]
    sx: np.ndarray       # fp16 [M, K/64]
    xl1: np.ndarray      # fp32 [M, r]


def quantize_act(x_bits: np.ndarray, inv_lambda, l1_bits) -> QuantAct:
    """x_hat = fp32(x) * inv_lambda (one fp32 multiply); xl1 = fp32(sum_k x_hat
    L1) accumulated in fp64; Qsym64 on every (row, group) of x_hat."""
    x = bf16_bits_to_f32(x_bits)
    M, K = x.shape
    inv = np.ones(K, np.float32) if inv_lambda is None else np.asarray(inv_lambda, np.float32)
    x_hat = (x * inv[None, :]).astype(np.float32)
    if l1_bits is None or np.asarray(l1_bits).shape[1] == 0:
        xl1 = np.zeros((M, 0), np.float32)
    else:
        l1 = bf16_bits_to_f32(l1_bits).astype(np.float64)
        xl1 = (x_hat.astype(np.float64) @ l1).astype(np.float32)
    codes, sx = quantize_rows(x_hat)
    return QuantAct(x_hat, codes, pack_int4(codes), sx, xl1)


def group_partials(qx_codes: np.ndarray, qw_codes: np.ndarray) -> np.ndarray:
    """P[m, n, g] = sum_{k in group g} qx[m, k] * qw[n, k], exact integers.
    Each group's product of integer codes is formed by a float64 matmul, which
    is exact here (|terms| <= 49, |sums| <= 64 * 49 < 2**53)."""
    a = group_view(np.asarray(qx_codes, np.int8))
    b = group_view(np.asarray(qw_codes, np.int8))
    G = a.shape[1]
    P = np.empty((a.shape[0], b.shape[0], G), np.int32)
    for g in range(G):
        P[:, :, g] = (a[:, g, :].astype(np.float64) @ b[:, g, :].astype(np.float64).T).astype(np.int32)
    return P


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    """0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))), fp64."""
    y = np.asarray(y, np.float64)
    return 0.5 * y * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (y + 0.044715 * y ** 3)))


def linear_output(qx_codes, sx, qw_codes, sw, xl1, l2_bits, bias_bits=None,
                  act: str = "none") -> np.ndarray:
    """Y64[m, n] = sum_g sx[m,g] sw[n,g] P_g[m,n] + sum_j xl1[m,j] L2[j,n] + bias[n],
    then GELU(tanh) if requested; all in fp64."""
    a = group_view(np.asarray(qx_codes, np.int8))
    b = group_view(np.asarray(qw_codes, np.int8))
    sxf = np.asarray(sx, np.float16).astype(np.float64)
    swf = np.asarray(sw, np.float16).astype(np.float64)
    M, G, _ = a.shape
    N = b.shape[0]
    y = np.zeros((M, N), np.float64)
    for g in range(G):
        p = a[:, g, :].astype(np.float64) @ b[:, g, :].astype(np.float64).T
        y += sxf[:, g][:, None] * swf[:, g][None, :] * p
    if xl1 is not None and np.asarray(xl1).shape[1] > 0:
        y += np.asarray(xl1, np.float64) @ bf16_bits_to_f32(l2_bits).astype(np.float64)
    if bias_bits is not None:
        y += bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    if act == "gelu_tanh":
        y = gelu_tanh(y)
    elif act != "none":
        raise ValueError(act)
    return y


def output_bf16(y64: np.ndarray) -> np.ndarray:
    return f64_to_bf16_bits(y64)


def forward(weights: SvdqWeights, x_bits: np.ndarray, act: str = "none"):
    """Online path for one batch of tokens: returns (QuantAct, Y64)."""
    qa = quantize_act(x_bits, weights.inv_lambda, weights.l1 if weights.rank else None)
    y = linear_output(qa.codes, qa.sx, weights.qw_codes, weights.sw, qa.xl1,
                      weights.l2, weights.bias, act)
    return qa, y


def exact_output(x_bits, w_bits, bias_bits=None) -> np.ndarray:
    """Diagnostic: the unquantised layer X W + bias in fp64."""
    y = bf16_bits_to_f32(x_bits).astype(np.float64) @ bf16_bits_to_f32(w_bits).astype(np.float64)
    if bias_bits is not None:
        y += bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return y


__all__ = [n for n in dir() if not n.startswith("_")] + ["f16_bits", "f16_from_bits",
                                                          "f32_to_bf16_bits"]
