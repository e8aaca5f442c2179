"""The offline quantiser on the GPU, as one call per layer: a bf16 weight
(and calibration activations) in, the arrays of an SVDQ layer out.

This is the Quantize step of the tool chain on the donmalab.com page
(section on quantising a model yourself: inspect, quantize, package,
validate); the remio.ai page (section on SVDQuant moving hard values out of
4-bit) gives the roles: calibration statistics set the smoothing, a 16-bit
low-rank branch takes the hardest part of the smoothed weight, and the
residual becomes 4-bit.

Marshalling only: every step is a library kernel (include/svdq.h, offline
quantiser); this module allocates the outputs and the fp64 scratch with
torch and calls the entry points in order on one stream. The random test
matrix of the range finder is drawn on the host from numpy's default
generator with the given seed (standard normal, N x l), the same draw the
oracle makes, and passed in.
"""
from __future__ import annotations

from typing import Iterable

import numpy as np
import torch

from . import _lib

LMAX = 88            # widest block the library's range finder takes


def block_width(K: int, N: int, rank: int, oversample: int = 16) -> int:
    """l = min(rank + oversample, K, N, LMAX): the range finder's block width."""
    return min(rank + oversample, K, N, LMAX)


def quantize_layer(w: torch.Tensor, x_calib, rank: int, alpha: float = 0.5, bias=None,
                   power_iters: int = 4, oversample: int = 16, seed: int = 0, smooth: bool = True,
                   omega=None, keep_factors: bool = False, fmt: str = "int4", stream=None) -> dict:
    """w: bf16 [K, N] on the GPU (K a multiple of 64, N of 8); x_calib: one
    bf16 [M, K] calibration batch or an iterable of them (None with
    smooth=False); fmt "int4" (symmetric INT4, fp16 scale per 64) or "mxfp4"
    (E2M1 codes, E8M0 exponent per 32; the same smoothing and low-rank
    branch). Returns the layer's device arrays: inv_lambda fp32 [K], l1t
    (tile layout), l2t bf16 [N, r], qw uint8 [N, K/2], sw (INT4: fp16
    [ceil(K/256), N, 4]; MXFP4: uint8 exponent records [ceil(K/256), N, 8]),
    bias, rank, fmt; with keep_factors also l1 [K, r], l2 [r, N] (bf16),
    sigma fp64 [r], w_hat fp64 [K, N]."""
    _lib._check_rows(w, "w", torch.bfloat16)
    K, N = w.shape
    dev = w.device
    _lib._require(K % 64 == 0 and N % 8 == 0, f"w must be [K, N] with K % 64 == 0 and N % 8 == 0, got {(K, N)}")
    _lib._require(rank == 0 or (rank % 16 == 0 and 16 <= rank <= 80), f"rank {rank} must be 0 or a multiple of 16 up to 80")
    _lib._require(fmt in ("int4", "mxfp4"), f"fmt must be 'int4' or 'mxfp4', got {fmt!r}")
    out = {}
    if smooth:
        _lib._require(x_calib is not None, "calibration activations are required when smoothing")
        batches: Iterable = [x_calib] if isinstance(x_calib, torch.Tensor) else x_calib
        ax = torch.empty(K, dtype=torch.float32, device=dev)
        first = True
        for xb in batches:
            _lib._check_rows(xb, "x_calib", torch.bfloat16)
            _lib._require(xb.shape[1] == K, f"calibration batch must have K = {K} columns")
            _lib._check_same_device(w, x_calib=xb)
            _lib.svdq_calib_absmax(xb, xb.shape[0], K, xb.stride(0), 0, 0 if first else 1, ax, stream)
            first = False
        _lib._require(not first, "no calibration batch given")
        aw = torch.empty(K, dtype=torch.float32, device=dev)
        _lib.svdq_calib_absmax(w, K, N, w.stride(0), 1, 0, aw, stream)
        inv_lambda = torch.empty(K, dtype=torch.float32, device=dev)
        _lib.svdq_smoothing(ax, aw, K, alpha, inv_lambda, stream)
        out.update(ax=ax, aw=aw)
    else:
        inv_lambda = torch.ones(K, dtype=torch.float32, device=dev)
    w_hat = torch.empty((K, N), dtype=torch.float64, device=dev)
    _lib.svdq_smooth_weight(w, K, N, w.stride(0), inv_lambda, w_hat, stream)
    l1 = torch.zeros((K, rank), dtype=torch.bfloat16, device=dev)
    l2 = torch.zeros((rank, N), dtype=torch.bfloat16, device=dev)
    sigma = torch.zeros(rank, dtype=torch.float64, device=dev)
    if rank:
        l = block_width(K, N, rank, oversample)
        if omega is None:
            om = np.random.default_rng(seed).standard_normal((N, min(rank + oversample, min(K, N))))
            _lib._require(om.shape[1] == l, f"the oracle's block width {om.shape[1]} exceeds {LMAX}")
            omega = torch.from_numpy(om).to(dev)
        _lib._require(omega.dtype == torch.float64 and tuple(omega.shape) == (N, l) and omega.is_contiguous(),
                      f"omega must be contiguous fp64 [{N}, {l}]")
        nbytes = _lib.svdq_lowrank_workspace_size(K, N, rank, l)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _lib.svdq_lowrank(w_hat, K, N, rank, omega, l, power_iters, l1, l2, sigma, ws, nbytes, stream)
    G4 = (K // 64 + 3) // 4
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if fmt == "int4":
        sw = torch.empty((G4, N, 4), dtype=torch.float16, device=dev)
        _lib.svdq_quantize_residual(w_hat, K, N, l1 if rank else None, l2 if rank else None, rank, qw, sw, stream)
    else:
        sw = torch.empty((G4, N, 8), dtype=torch.uint8, device=dev)
        _lib.svdq_quantize_residual_mxfp4(w_hat, K, N, l1 if rank else None, l2 if rank else None, rank, qw, sw,
                                          stream)
    l1t = torch.empty(K * rank, dtype=torch.bfloat16, device=dev)
    l2t = torch.empty((N, rank), dtype=torch.bfloat16, device=dev)
    _lib.svdq_pack_lowrank(l1, l2, K, N, rank, l1t, l2t, stream)
    out.update(inv_lambda=inv_lambda, l1t=l1t, l2t=l2t, qw=qw, sw=sw, bias=bias, rank=rank, fmt=fmt)
    if keep_factors:
        out.update(l1=l1, l2=l2, sigma=sigma, w_hat=w_hat)
    return out


def quantize_awq(w: torch.Tensor, inv_s=None, stream=None) -> dict:
    """The AWQ W4A16 weight quantisation on the GPU: w bf16 [K, N] (K a
    multiple of 128, N of 16; rows may be strided), inv_s fp32 [K] (the
    reciprocal activation-aware channel scales) or None. Returns the operands
    of awq_gemv in its tile layouts: qwt uint8 [N * K / 2], scale_t and
    zero_t fp16 [N * K / 64], and inv_s."""
    _lib._check_rows(w, "w", torch.bfloat16)
    K, N = w.shape
    dev = w.device
    _lib._require(K % 128 == 0 and N % 16 == 0, f"w must be [K, N] with K % 128 == 0 and N % 16 == 0, got {(K, N)}")
    if inv_s is not None:
        _lib._require(inv_s.dtype == torch.float32 and inv_s.numel() == K and inv_s.is_contiguous(),
                      f"inv_s must be a contiguous fp32 vector of K = {K} values")
        _lib._check_same_device(w, inv_s=inv_s)
    qwt = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    scale_t = torch.empty(N * K // 64, dtype=torch.float16, device=dev)
    zero_t = torch.empty(N * K // 64, dtype=torch.float16, device=dev)
    _lib.awq_quantize_weight(w, K, N, w.stride(0), inv_s, qwt, scale_t, zero_t, stream)
    return dict(qwt=qwt, scale_t=scale_t, zero_t=zero_t, inv_s=inv_s, K=K, N=N)
