"""GPU parity of the MXFP4 form of the SVDQ layer against the CPU oracle
(oracle/mxfp4.py), through the C ABI.

Bars: E2M1 codes and E8M0 exponents bit-exact; xl1 relative Frobenius error
<= 1e-4; fp32 output element-wise within the fp32 accumulation bound of the
fp64 definition and within 1e-5 relative Frobenius; bf16 output the RTNE of
the same kernel's fp32 output and within the 2e-3 relative Frobenius gate.
"""
import functools

import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4 as omx, numfmt, svdq as osv
from gpu_util import (assert_bf16_is_rounded_fp32, assert_fp32_gelu, dev, dev_u16, host_bf16_f64,
                      host_u16, note, rel_fro, sample_rows)

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib


class DevMx:
    """Oracle-prepared MXFP4 layer in the library's layouts."""

    def __init__(self, w):
        self.w = w
        self.rank = w.rank
        self.inv_lambda = dev(w.inv_lambda)
        self.l1t = dev_u16(osv.pack_l1_tiles(w.l1)) if w.rank else None
        self.l2t = dev_u16(np.ascontiguousarray(w.l2.T)) if w.rank else None
        self.qw = dev(omx.pack_fp4(w.qw_codes))
        self.sw = dev(omx.pack_scales(w.qw_exps))
        self.bias = dev_u16(w.bias) if w.bias is not None else None


@functools.lru_cache(maxsize=None)
def layer(name, M=None):
    cfg = synth.CONFIGS[name]
    li = synth.make_layer(cfg, M=M)
    w = omx.prepare_mx(li.x, li.w, li.bias, cfg.rank)
    return cfg, li, w


def check_act(qa, qx, sx, xl1, rank):
    assert np.array_equal(qx.cpu().numpy(), omx.pack_fp4(qa.codes)), "E2M1 codes differ"
    assert np.array_equal(sx.cpu().numpy(), omx.pack_scales(qa.exps)), "E8M0 exponents differ"
    if rank:
        e = rel_fro(xl1.cpu().numpy(), qa.xl1)
        assert e <= 1e-4, e


def magnitude(qa_codes, qa_exps, w_codes, w_exps, xl1, l2_bits, bias_bits):
    """(T, T_lr): the sum of |terms| per output (the scale of the fp32
    accumulation error) and its low-rank part alone (whose fp32 input xl1 the
    GPU splits into bf16 hi + lo, which keeps 16-17 bits)."""
    a = np.abs(omx.dequantize_rows(qa_codes, qa_exps))
    w = np.abs(omx.dequantize_rows(w_codes, w_exps))
    t = a @ w.T
    t_lr = np.zeros_like(t)
    if xl1 is not None and xl1.shape[1]:
        t_lr = np.abs(xl1.astype(np.float64)) @ np.abs(numfmt.bf16_bits_to_f32(l2_bits).astype(np.float64))
        t += t_lr
    if bias_bits is not None:
        t += np.abs(numfmt.bf16_bits_to_f32(bias_bits).astype(np.float64))[None, :]
    return t, t_lr


def fp32_bound_mx(tmag, K, rank):
    # fp32 sums of K / 64 MFMA steps, the low-rank MFMAs, bias: a few ulps of
    # the magnitude per term that meets the accumulator; plus the residual of
    # the bf16 hi/lo split of the low-rank input (as for the INT4 form)
    t, t_lr = tmag
    return 2.0 * (K // 64 + rank + 4) * 2.0 ** -24 * t + 2.0 ** -16 * t_lr


def assert_fp32(y32, y64, tmag, K, rank):
    bound = fp32_bound_mx(tmag, K, rank)
    assert np.all(np.abs(y32 - y64) <= bound + 1e-30), float(np.max(np.abs(y32 - y64) - bound))
    assert rel_fro(y32, y64) <= 1e-5


@pytest.mark.parametrize("name,M", [("tiny", None), ("tiny", 77), ("qkv", None)])
def test_mx_act_parity(name, M):
    note(f"mxfp4 act {name} M={M}")
    cfg, li, w = layer(name, M)
    dw = DevMx(w)
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(li.x), dw.inv_lambda, dw.l1t, cfg.rank)
    torch.cuda.synchronize()
    qa = omx.quantize_act(li.x, w.inv_lambda, w.l1)
    check_act(qa, qx, sx, xl1, cfg.rank)


@pytest.mark.parametrize("M,K,rank", [(300, 12800, 32), (50, 3200, 16), (4645, 3072, 32)], ids=lambda v: str(v))
def test_mx_act_ring_paths(M, K, rank):
    """The launch shapes of the LDS-staged kernel (ring loop with uneven
    group counts per wave, conditional last-round requests, more row blocks
    than CUs with a ragged last block)."""
    note(f"mxfp4 act ring M={M} K={K} rank={rank}")
    x = synth.make_matrix_bf16(M, K, seed=K + rank + 1, std=1.5)
    rng = np.random.default_rng(K + 1)
    inv = rng.uniform(0.3, 2.5, K).astype(np.float32)
    l1 = numfmt.f32_to_bf16_bits((rng.standard_normal((K, rank)) * 0.05).astype(np.float32))
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(x), dev(inv), dev_u16(osv.pack_l1_tiles(l1)), rank)
    torch.cuda.synchronize()
    qa = omx.quantize_act(x, inv, l1)
    check_act(qa, qx, sx, xl1, rank)


def test_mx_act_edge_values():
    """Exact E2M1 ties, saturation, zero blocks, tiny and clamped exponents."""
    note("mxfp4 act edge values")
    M, K = 16, 320                                   # 10 blocks: a padded scale quad
    rng = np.random.default_rng(4)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[0] = 0.0
    xf[1, :32] = 0.0
    xf[2, :10] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0]
    xf[2, 10:32] = 0.0
    xf[3, :32] = np.linspace(-7.9, 7.9, 32)          # amax < 8: values above 6 saturate
    xf[4] *= 1e-30
    xf[5, :32] *= 2.0 ** -125                        # exponent clamps at -127
    xf[6] *= 1e30
    xbits = numfmt.f32_to_bf16_bits(xf)
    qx, sx, _ = lib.quantize_act_mxfp4(dev_u16(xbits), None, None, 0)
    torch.cuda.synchronize()
    qa = omx.quantize_act(xbits, None, None)
    check_act(qa, qx, sx, None, 0)


@pytest.mark.parametrize("act,bias", [("none", True), ("gelu_tanh", True), ("none", False)])
def test_mx_gemm_tiny(act, bias):
    note(f"mxfp4 gemm tiny act={act} bias={bias}")
    cfg, li, w = layer("tiny")
    dw = DevMx(w)
    qa = omx.quantize_act(li.x, w.inv_lambda, w.l1)
    qxd, sxd, xld = dev(omx.pack_fp4(qa.codes)), dev(omx.pack_scales(qa.exps)), dev(qa.xl1)
    b = dw.bias if bias else None
    bb = w.bias if bias else None
    y32 = lib.mxfp4_linear(qxd, sxd, xld, dw.qw, dw.sw, dw.l2t, b, cfg.rank, act=act, out_dtype=torch.float32)
    ybf = lib.mxfp4_linear(qxd, sxd, xld, dw.qw, dw.sw, dw.l2t, b, cfg.rank, act=act)
    torch.cuda.synchronize()
    y64 = omx.linear_output(qa.codes, qa.exps, w.qw_codes, w.qw_exps, qa.xl1, w.l2, bb, act)
    y32h = y32.cpu().numpy()
    tmag = magnitude(qa.codes, qa.exps, w.qw_codes, w.qw_exps, qa.xl1, w.l2, bb)
    if act == "none":
        assert_fp32(y32h, y64, tmag, cfg.K, cfg.rank)
    else:
        pre64 = omx.linear_output(qa.codes, qa.exps, w.qw_codes, w.qw_exps, qa.xl1, w.l2, bb, "none")
        assert_fp32_gelu(y32h, pre64, fp32_bound_mx(tmag, cfg.K, cfg.rank))
    assert_bf16_is_rounded_fp32(host_u16(ybf), y32h)
    assert rel_fro(host_bf16_f64(ybf), y64) <= 2e-3


def test_mx_gemm_ragged_and_ranks():
    """Ragged M and N against the tile, rank 0, the maximum rank, a half rank
    chunk, rank 64 (ranks above 32 take the register form of the activation
    kernel and several low-rank chunks in the GEMM), one row with one group,
    and K with a partly filled scale quad."""
    for (M, K, N, r) in [(77, 192, 200, 0), (130, 320, 136, 128), (300, 704, 264, 48), (1, 64, 16, 16),
                         (64, 512, 96, 64)]:
        note(f"mxfp4 ragged M={M} K={K} N={N} r={r}")
        x = synth.make_matrix_bf16(M, K, seed=M, std=1.0)
        wb = synth.make_matrix_bf16(K, N, seed=N, std=0.05)
        b = synth.make_matrix_bf16(1, N, seed=3, std=0.02)[0]
        w = omx.prepare_mx(x, wb, b, r)
        dw = DevMx(w)
        qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(x), dw.inv_lambda, dw.l1t, r)
        y = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, r, out_dtype=torch.float32)
        ybf = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, r)
        torch.cuda.synchronize()
        qa, y64 = omx.forward(w, x)
        check_act(qa, qx, sx, xl1, r)
        tmag = magnitude(qa.codes, qa.exps, w.qw_codes, w.qw_exps, qa.xl1 if r else None, w.l2, w.bias)
        assert_fp32(y.cpu().numpy(), y64, tmag, K, r)
        assert_bf16_is_rounded_fp32(host_u16(ybf), y.cpu().numpy())


def test_mx_qkv_full_size():
    """The QKV shape end to end (act + GEMM, the launches the benchmark
    times): every code and exponent compared; outputs on sampled rows."""
    note("mxfp4 qkv full size")
    cfg, li, w = layer("qkv")
    dw = DevMx(w)
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(li.x), dw.inv_lambda, dw.l1t, cfg.rank)
    y = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank)
    yf = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa = omx.quantize_act(li.x, w.inv_lambda, w.l1)
    check_act(qa, qx, sx, xl1, cfg.rank)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(cfg.M - 8, cfg.M),
                                     np.random.default_rng(0).choice(cfg.M, 40, replace=False)]))
    y64 = omx.linear_output(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows],
                            w.l2, w.bias)
    tmag = magnitude(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows], w.l2, w.bias)
    assert_fp32(yf.cpu().numpy()[rows], y64, tmag, cfg.K, cfg.rank)
    assert_bf16_is_rounded_fp32(host_u16(y), yf.cpu().numpy())
    assert rel_fro(host_bf16_f64(y)[rows], y64) <= 2e-3


def test_mx_fused_projection_column_split():
    """The fused-projection column split on the MXFP4 layer (QKV size)."""
    note("mxfp4 fused projection split qkv")
    cfg, li, w = layer("qkv")
    dw = DevMx(w)
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(li.x), dw.inv_lambda, dw.l1t, cfg.rank)
    sizes = (3072, 3072, 3072)
    y = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank)
    parts = lib.projection_weights(dw.qw, dw.sw, dw.l2t, dw.bias, sizes)
    ys = [lib.mxfp4_linear(qx, sx, xl1, q, s, l2, b, cfg.rank) for (q, s, l2, b) in parts]
    torch.cuda.synchronize()
    for view, yp in zip(lib.split_columns(y, sizes), ys):
        assert torch.equal(view.contiguous().view(torch.int16), yp.view(torch.int16))


def test_mx_act_strided_rows():
    """MXFP4 activation kernel on rows with a leading dimension beyond K."""
    note("mxfp4 act ldx > K")
    M, K, r, pad = 70, 320, 32, 64
    xw = synth.make_matrix_bf16(M, K + pad, seed=13, std=1.5)
    x = np.ascontiguousarray(xw[:, 32:32 + K])
    rng = np.random.default_rng(14)
    inv = rng.uniform(0.3, 2.0, K).astype(np.float32)
    l1 = numfmt.f32_to_bf16_bits((rng.standard_normal((K, r)) * 0.1).astype(np.float32))
    xd = dev_u16(xw)[:, 32:32 + K]
    qx, sx, xl1 = lib.quantize_act_mxfp4(xd, dev(inv), dev_u16(osv.pack_l1_tiles(l1)), r)
    torch.cuda.synchronize()
    qa = omx.quantize_act(x, inv, l1)
    check_act(qa, qx, sx, xl1, r)


def test_mx_fc2_full_size():
    """The MXFP4 block's longest-K layer at full size: fc2, 4608 x 12288 ->
    3072, rank 32 (a seeded stand-in for the GELU output as input). Every
    code and exponent of the activation pass; outputs on sampled rows."""
    note("mxfp4 fc2 full size")
    c2 = synth.CONFIGS["mlp_fc2"]
    li = synth.make_layer(c2, M=8)                   # fc2's weights and bias
    x = synth.make_matrix_bf16(c2.M, c2.K, seed=31, std=0.4)
    w = omx.prepare_mx(x, li.w, li.bias, c2.rank)
    dw = DevMx(w)
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(x), dw.inv_lambda, dw.l1t, c2.rank)
    y = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, c2.rank)
    yf = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, c2.rank, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa = omx.quantize_act(x, w.inv_lambda, w.l1)
    check_act(qa, qx, sx, xl1, c2.rank)
    rows = sample_rows(c2.M, 4, 24, 2)
    y64 = omx.linear_output(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows],
                            w.l2, w.bias)
    tmag = magnitude(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows], w.l2, w.bias)
    yfh = yf.cpu().numpy()
    assert_fp32(yfh[rows], y64, tmag, c2.K, c2.rank)
    assert_bf16_is_rounded_fp32(host_u16(y), yfh)
    assert rel_fro(host_bf16_f64(y)[rows], y64) <= 2e-3


@pytest.mark.parametrize("K,N,act", [(3072, 3072, "none"), (3072, 12288, "gelu_tanh")],
                         ids=["out_proj", "fc1_gelu"])
def test_mx_block_layers_full_size(K, N, act):
    """The MXFP4 block's out-projection (3072 -> 3072) and fc1 with the GELU
    epilogue (3072 -> 12288) at 4608 tokens, rank 32: every code and exponent
    of the activation pass; fp32 outputs element-wise on sampled rows (GELU:
    the pre-activation bound carried through GELU), bf16 = RTNE of fp32."""
    M, R = 4608, 32
    note(f"mxfp4 block layer K={K} N={N} act={act}")
    cfg = synth.LayerConfig("blk", M=M, K=K, N=N, rank=R, n_outliers=31, outlier_factor=30.0,
                            seed=K + N)
    li = synth.make_layer(cfg)
    w = omx.prepare_mx(li.x, li.w, li.bias, R)
    dw = DevMx(w)
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(li.x), dw.inv_lambda, dw.l1t, R)
    y = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, R, act=act)
    yf = lib.mxfp4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, R, act=act, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa = omx.quantize_act(li.x, w.inv_lambda, w.l1)
    check_act(qa, qx, sx, xl1, R)
    rows = sample_rows(M, 4, 24, 3)
    pre = omx.linear_output(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows], w.l2, w.bias)
    tmag = magnitude(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows], w.l2, w.bias)
    yfh = yf.cpu().numpy()
    if act == "none":
        assert_fp32(yfh[rows], pre, tmag, K, R)
        y64 = pre
    else:
        assert_fp32_gelu(yfh[rows], pre, fp32_bound_mx(tmag, K, R))
        y64 = omx.linear_output(qa.codes[rows], qa.exps[rows], w.qw_codes, w.qw_exps, qa.xl1[rows], w.l2,
                                w.bias, act)
    assert_bf16_is_rounded_fp32(host_u16(y), yfh)
    assert rel_fro(host_bf16_f64(y)[rows], y64) <= 2e-3
