"""MXFP4 variant of the SVDQ W4A4 layer (oracle; test infrastructure only:
imported by tests/, __graft_entry__.smoke() and bench.py's CPU baseline,
never by the library).

The pages run the SVDQ layer with 4-bit INT codes on older NVIDIA parts and
with NVFP4 on Blackwell (remio.ai page, loading-path and benchmark sections);
they do not describe a microscaled format for other hardware. This variant
keeps every step of the method (smoothing, low-rank branch, 4-bit residual
and 4-bit activations, sum of the two) and only replaces the 4-bit number
format by OCP MXFP4, whose definition is taken from the OCP Microscaling
Formats (MX) Specification v1.0 (the E2M1 element type, the E8M0 scale type
and the conversion of FP32 vectors to an MX format):

  * a block is 32 consecutive values along K (per token row for X_hat, per
    output column for the residual R);
  * the block's shared exponent is e = floor(log2(amax)) - 2, where 2 is the
    exponent of the largest E2M1 normal (6 = 1.5 * 2^2); e is clamped to
    the E8M0 range [-127, 127]; a block of zeros gets e = -127;
  * each element is v / 2^e rounded to the nearest E2M1 value, ties to the
    value whose mantissa bit is 0, magnitudes beyond 6 saturating to 6.

Readings where the spec leaves a choice to the implementation: a result of
zero is stored with sign 0 (as the INT4 format does); scales are stored as
E8M0 bytes e + 127 in a quad-major layout (below).

Storage (library format v3, MXFP4 side):
  * codes: one nibble per value, bit 3 sign, bits 0-2 the index of the
    magnitude in E2M1_GRID (which is the E2M1 exponent/mantissa encoding);
    element 2i of a row in bits 0-3 of byte i, element 2i + 1 in bits 4-7;
    weights transposed [N][K/2];
  * scales: E8M0 bytes in an array [ceil(K/256)][rows][8]: the 8 bytes of
    (quad q, row r) hold the exponents of blocks 8q .. 8q + 7 of the row,
    even blocks first: byte h * 4 + j is block 8q + 2j + h; blocks past
    K/32 hold 0.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import svdq
from .numfmt import bf16_bits_to_f32

BLOCK = 32
EMAX_ELEM = 2                       # exponent of the largest E2M1 normal
E8M0_MIN, E8M0_MAX = -127, 127
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def e2m1_round(t) -> np.ndarray:
    """Round values to E2M1 magnitudes with sign: returns signed codes in
    [-7, 7] (sign * index into E2M1_GRID). Nearest value, ties to the even
    index (mantissa bit 0), |t| > 6 saturates; zero results carry sign 0."""
    t = np.asarray(t, np.float64)
    a = np.abs(t)
    idx = np.zeros(a.shape, np.int64)
    for k in range(1, len(E2M1_GRID)):
        lo, hi = E2M1_GRID[k - 1], E2M1_GRID[k]
        mid = 0.5 * (lo + hi)
        up = (a > mid) | ((a == mid) & (k % 2 == 0))   # tie: the even index wins
        idx = np.where(up, k, idx)
    idx = np.where(a > E2M1_MAX, 7, idx)
    return np.where((t < 0) & (idx > 0), -idx, idx).astype(np.int8)


def block_exponent(amax) -> np.ndarray:
    """Shared exponent of blocks with the given absolute maxima."""
    amax = np.asarray(amax, np.float64)
    _, e2 = np.frexp(amax)                   # amax = m * 2**e2, m in [0.5, 1)
    e = (e2 - 1) - EMAX_ELEM                 # floor(log2(amax)) - emax_elem
    e = np.clip(e, E8M0_MIN, E8M0_MAX)
    return np.where(amax > 0, e, E8M0_MIN).astype(np.int16)


def quantize_rows(v_f32: np.ndarray):
    """MXFP4 quantisation of every 32-block of a [rows, K] float32 matrix.
    Returns (signed codes int8 [rows, K], exponents int16 [rows, K/32])."""
    v = np.asarray(v_f32, np.float32).astype(np.float64)
    rows, K = v.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    b = v.reshape(rows, K // BLOCK, BLOCK)
    e = block_exponent(np.abs(b).max(axis=2))
    t = b / np.ldexp(1.0, e.astype(np.int64))[..., None]      # exact: power of two
    return e2m1_round(t).reshape(rows, K), e


def dequantize_rows(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.int64)
    mag = E2M1_GRID[np.abs(c)] * np.sign(c)
    rows, K = c.shape
    return (mag.reshape(rows, K // BLOCK, BLOCK)
            * np.ldexp(1.0, np.asarray(exps, np.int64))[..., None]).reshape(rows, K)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Signed codes [rows, K] -> nibbles [rows, K/2] (sign bit 3, index bits 0-2)."""
    c = np.asarray(codes, np.int16)
    if c.min(initial=0) < -7 or c.max(initial=0) > 7:
        raise ValueError("codes out of [-7, 7]")
    rows, K = c.shape
    if K % 2:
        raise ValueError("K must be even")
    nib = (np.abs(c) | np.where(c < 0, 8, 0)).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    nib = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    nib[:, 0::2] = p & 15
    nib[:, 1::2] = p >> 4
    mag = (nib & 7).astype(np.int8)
    return np.where(nib & 8, -mag, mag).astype(np.int8)


def pack_scales(exps: np.ndarray) -> np.ndarray:
    """Exponents [rows, K/32] -> E8M0 bytes [ceil(K/256)][rows][8] (see the
    module docstring for the order inside a quad)."""
    e = np.asarray(exps, np.int64)
    rows, nb = e.shape
    nq = (nb + 7) // 8
    out = np.zeros((nq, rows, 8), np.uint8)
    for b in range(nb):
        q, bl = divmod(b, 8)
        out[q, :, (bl % 2) * 4 + bl // 2] = (e[:, b] + 127).astype(np.uint8)
    return out


def unpack_scales(packed: np.ndarray, nblocks: int) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty((p.shape[1], nblocks), np.int16)
    for b in range(nblocks):
        q, bl = divmod(b, 8)
        out[:, b] = p[q, :, (bl % 2) * 4 + bl // 2].astype(np.int16) - 127
    return out


@dataclass
class MxWeights:
    K: int
    N: int
    rank: int
    inv_lambda: np.ndarray   # fp32 [K]
    l1: np.ndarray           # bf16 bits [K, r]
    l2: np.ndarray           # bf16 bits [r, N]
    qw_codes: np.ndarray     # int8 [N, K]
    qw_exps: np.ndarray      # int16 [N, K/32]
    bias: np.ndarray | None  # bf16 bits [N]


def prepare_mx(x_bits, w_bits, bias_bits, rank: int, alpha: float = 0.5, svd_seed: int = 0) -> MxWeights:
    """Offline preparation as for the INT4 layer (calibration, smoothing,
    low-rank factors, residual), the residual quantised to MXFP4 per output
    column."""
    x = bf16_bits_to_f32(x_bits)
    w = bf16_bits_to_f32(w_bits)
    K, N = w.shape
    ax, aw = svdq.calib_absmax(x, w)
    _, inv_lam = svdq.smoothing(ax, aw, alpha)
    w_hat = svdq.smooth_weight(w, inv_lam)
    l1, l2, _ = svdq.lowrank_factors(w_hat, rank, seed=svd_seed)
    r = svdq.residual(w_hat, l1, l2)
    codes, exps = quantize_rows(np.ascontiguousarray(r.T))
    return MxWeights(K, N, rank, inv_lam, l1, l2, codes, exps,
                     None if bias_bits is None else np.asarray(bias_bits, np.uint16))


@dataclass
class MxAct:
    x_hat: np.ndarray    # fp32 [M, K]
    codes: np.ndarray    # int8 [M, K]
    exps: np.ndarray     # int16 [M, K/32]
    xl1: np.ndarray      # fp32 [M, r]


def quantize_act(x_bits, inv_lambda, l1_bits) -> MxAct:
    """x_hat and xl1 exactly as the INT4 layer computes them; MXFP4 codes and
    exponents of x_hat."""
    qa = svdq.quantize_act(x_bits, inv_lambda, l1_bits)
    codes, exps = quantize_rows(qa.x_hat)
    return MxAct(qa.x_hat, codes, exps, qa.xl1)


def linear_output(a_codes, a_exps, w_codes, w_exps, xl1, l2_bits, bias_bits=None,
                  act: str = "none") -> np.ndarray:
    """Y64 = deq(A) deq(W)^T + xl1 L2 + bias (then GELU if requested), fp64.
    Every dequantised value is exact in fp64 (E2M1 value times a power of
    two), and so is each product; the matmul is the library primitive."""
    a = dequantize_rows(a_codes, a_exps)
    w = dequantize_rows(w_codes, w_exps)
    y = a @ w.T
    if xl1 is not None and np.asarray(xl1).shape[1] > 0:
        y = y + np.asarray(xl1, np.float64) @ bf16_bits_to_f32(l2_bits).astype(np.float64)
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    if act == "gelu_tanh":
        y = svdq.gelu_tanh(y)
    return y


def forward(w: MxWeights, x_bits, act: str = "none"):
    qa = quantize_act(x_bits, w.inv_lambda, w.l1)
    return qa, linear_output(qa.codes, qa.exps, w.qw_codes, w.qw_exps, qa.xl1, w.l2, w.bias, act)
