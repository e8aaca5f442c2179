"""Shared helpers for the GPU parity tests: moving oracle arrays to the
device in the library's layouts, and error measures."""
from __future__ import annotations

import sys

import numpy as np
import torch


def note(msg: str):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(dtype).cuda()


def dev_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float16))).cuda()


def dev_scales(s: np.ndarray) -> torch.Tensor:
    """fp16 group scales [rows, G] -> the device array in the library's
    quad-major layout [ceil(G/4)][rows][4]."""
    from oracle import svdq as osv
    return dev_f16(osv.pack_scales(s))


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def host_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


class DevSvdq:
    """Oracle-prepared SVDQ layer moved to the device in the ABI layouts:
    L1 in the L1 tile layout, L2 as [N][r] (transposed)."""

    def __init__(self, w):
        from oracle import svdq as osv
        self.w = w
        self.rank = w.rank
        self.inv_lambda = dev(w.inv_lambda)
        self.l1t = dev_u16(osv.pack_l1_tiles(w.l1)) if w.rank else None
        self.l2t = dev_u16(np.ascontiguousarray(w.l2.T)) if w.rank else None
        self.qw = dev(w.qw)
        self.sw = dev_scales(w.sw)
        self.bias = dev_u16(w.bias) if w.bias is not None else None


def bf16_ulp(y64: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |y| (8 significant bits; subnormal floor)."""
    a = np.abs(np.asarray(y64, np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def assert_bf16_output(yg: np.ndarray, y64: np.ndarray, delta_rel: float):
    """Element-wise bar for a bf16 output against the fp64 definition: the GPU
    rounds its fp32 result once, so |yg - y64| <= ulp/2 of y64 plus the fp32
    accumulation error, bounded by delta_rel * rms(y64)."""
    yg = np.asarray(yg, np.float64)
    y64 = np.asarray(y64, np.float64)
    rms = float(np.sqrt(np.mean(y64 * y64)))
    bound = 0.5 * bf16_ulp(y64) * (1 + 2.0 ** -7) + delta_rel * rms
    bad = np.abs(yg - y64) > bound
    assert not bad.any(), (f"{bad.sum()} of {bad.size} elements outside ulp/2 + {delta_rel:g} rms; "
                           f"worst excess {np.max(np.abs(yg - y64) - bound):.3g}")
    assert rel_fro(yg, y64) <= 2e-3


def magnitude_sum(qx_codes, sx, qw_codes, sw, xl1, l2_bits, bias_bits):
    """(T, T_lr): T[m, n] = sum_g |sx sw P_g| + sum_j |xl1_j L2_jn| + |bias_n|,
    the scale of every term the fp32 accumulation adds, and T_lr the low-rank
    part alone (its fp32 input is split into bf16 hi + lo on the GPU, which
    keeps ~17 bits)."""
    from oracle import numfmt
    a = np.asarray(qx_codes, np.float64)
    b = np.asarray(qw_codes, np.float64)
    G = a.shape[1] // 64
    sxf = np.asarray(sx, np.float16).astype(np.float64)
    swf = np.asarray(sw, np.float16).astype(np.float64)
    t = np.zeros((a.shape[0], b.shape[0]))
    t_lr = np.zeros_like(t)
    for g in range(G):
        p = a[:, 64 * g:64 * g + 64] @ b[:, 64 * g:64 * g + 64].T
        t += np.abs(sxf[:, g][:, None] * swf[:, g][None, :] * p)
    if xl1 is not None and np.asarray(xl1).shape[1]:
        t_lr = np.abs(np.asarray(xl1, np.float64)) @ np.abs(numfmt.bf16_bits_to_f32(l2_bits).astype(np.float64))
        t += t_lr
    if bias_bits is not None:
        t += np.abs(numfmt.bf16_bits_to_f32(bias_bits).astype(np.float64))[None, :]
    return t, t_lr


def fp32_bound(tmag, n_terms: int):
    """Element-wise error allowance of the fp32 result: accumulation of n_terms
    terms, 2 (n_terms + 4) 2^-24 T, plus the hi/lo split residual of the
    low-rank input, 2^-16 T_lr (bf16 hi + bf16 lo keep 16-17 bits)."""
    t, t_lr = tmag
    return 2.0 * (n_terms + 4) * 2.0 ** -24 * t + 2.0 ** -16 * t_lr + 1e-30


def assert_fp32_output(y32, y64, tmag, n_terms: int):
    """|y32 - y64| <= fp32_bound element-wise, relative Frobenius <= 1e-5."""
    y32 = np.asarray(y32, np.float64)
    bound = fp32_bound(tmag, n_terms)
    bad = np.abs(y32 - y64) > bound
    assert not bad.any(), (f"{bad.sum()} of {bad.size} fp32 outputs outside the accumulation bound; "
                           f"worst ratio {np.max(np.abs(y32 - y64) / bound):.3g}")
    assert rel_fro(y32, y64) <= 1e-5


def assert_bf16_is_rounded_fp32(ybf_bits: np.ndarray, y32: np.ndarray):
    """The bf16 output is the RTNE rounding of the same kernel's fp32 result."""
    from oracle import numfmt
    exp = numfmt.f32_to_bf16_bits(np.asarray(y32, np.float32))
    assert np.array_equal(np.asarray(ybf_bits, np.uint16), exp)


def assert_fp32_gelu(y32, pre64, pre_bound):
    """fp32 output of the GELU epilogue against GELU(fp64 pre-activation):
    the pre-activation error (at most pre_bound, the fp32 accumulation bound)
    passes through GELU, whose slope never exceeds 1.13; evaluating GELU in
    fp32 adds a small relative error (allowed: 2^-18 of the value) and, in the
    far negative tail where GELU is below 1e-28 and its tanh form cancels,
    about an ulp of the input (allowed: 2^-22 of |pre|)."""
    from oracle import svdq as osv
    y32 = np.asarray(y32, np.float64)
    pre64 = np.asarray(pre64, np.float64)
    g64 = osv.gelu_tanh(pre64)
    bound = (1.13 * np.asarray(pre_bound, np.float64) + 2.0 ** -18 * np.abs(g64) + 2.0 ** -22 * np.abs(pre64)
             + 1e-30)
    bad = np.abs(y32 - g64) > bound
    assert not bad.any(), (f"{bad.sum()} of {bad.size} GELU outputs outside the bound; "
                           f"worst ratio {np.max(np.abs(y32 - g64) / bound):.3g}")
    assert rel_fro(y32, g64) <= 1e-5


def sample_rows(M: int, n_edge: int, n_rand: int, seed: int) -> np.ndarray:
    """First and last n_edge rows plus n_rand seeded random rows, sorted."""
    return np.unique(np.concatenate([np.arange(0, n_edge), np.arange(M - n_edge, M),
                                     np.random.default_rng(seed).choice(M, n_rand, replace=False)]))
