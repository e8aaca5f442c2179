"""GPU parity of the SVDQ W4A4 path against the CPU oracle, through the C ABI.

Bars: packed activation codes and fp16 scales bit-exact; per-group integer
partials bit-exact; xl1 relative Frobenius error <= 1e-4; fp32 output within
1e-5 (relative Frobenius) of the fp64 definition; bf16 output element-wise
within half a bf16 ulp of the fp64 value plus 1e-5 * rms (the fp32
accumulation error), and within the 2e-3 relative Frobenius gate.
"""
import functools

import numpy as np
import pytest
import torch

import synth
from oracle import numfmt, svdq as osv
from gpu_util import (DevSvdq, assert_bf16_is_rounded_fp32, assert_bf16_output, assert_fp32_gelu,
                      assert_fp32_output, dev, dev_f16, dev_scales, dev_u16, fp32_bound, host_bf16_f64,
                      host_u16, magnitude_sum, note, rel_fro, sample_rows)

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib


@functools.lru_cache(maxsize=None)
def layer(name, M=None):
    cfg = synth.CONFIGS[name]
    li = synth.make_layer(cfg, M=M)
    w = osv.prepare_svdq(li.x, li.w, li.bias, cfg.rank)
    return cfg, li, w


def run_act(x_bits, dw, rank):
    x = dev_u16(x_bits)
    return lib.quantize_act(x, dw.inv_lambda, dw.l1t, rank)


def check_act(qa, qx, sx, xl1, rank):
    assert np.array_equal(qx.cpu().numpy(), qa.qx), "packed codes differ"
    assert np.array_equal(sx.cpu().numpy().view(np.uint16),
                          osv.pack_scales(qa.sx).view(np.uint16)), "scales differ"
    if rank:
        e = rel_fro(xl1.cpu().numpy(), qa.xl1)
        assert e <= 1e-4, e


@pytest.mark.parametrize("name,M", [("tiny", None), ("qkv", None), ("tiny", 77), ("mlp_fc1", 4608)])
def test_act_quant_parity(name, M):
    note(f"act_quant {name} M={M}")
    cfg, li, w = layer(name, M)
    dw = DevSvdq(w)
    qx, sx, xl1 = run_act(li.x, dw, cfg.rank)
    torch.cuda.synchronize()
    qa = osv.quantize_act(li.x, w.inv_lambda, w.l1)
    check_act(qa, qx, sx, xl1, cfg.rank)


@pytest.mark.parametrize("rank,use_inv", [(0, False), (0, True), (32, False), (128, True)])
def test_act_quant_ranks_and_no_smoothing(rank, use_inv):
    note(f"act_quant rank={rank} inv={use_inv}")
    M, K = 45, 320
    x = synth.make_matrix_bf16(M, K, seed=5, std=2.0)
    rng = np.random.default_rng(6)
    inv = rng.uniform(0.2, 3.0, K).astype(np.float32) if use_inv else None
    l1 = numfmt.f32_to_bf16_bits((rng.standard_normal((K, rank)) * 0.1).astype(np.float32))
    xd = dev_u16(x)
    qx, sx, xl1 = lib.quantize_act(xd, dev(inv) if use_inv else None,
                                   dev_u16(osv.pack_l1_tiles(l1)) if rank else None, rank)
    torch.cuda.synchronize()
    qa = osv.quantize_act(x, inv, l1 if rank else None)
    check_act(qa, qx, sx, xl1, rank)


# Launch shapes of the LDS-staged activation kernel: K = 12800 (200 groups:
# waves with 13 and with 12 groups in the steady ring loop, 16 waves with two
# slots), K = 3200 (50 groups: a fourth group requested in the last round for
# two waves only), and 4645 rows (more row blocks than CUs: 8 waves, three
# slots, two workgroups per CU; a ragged last block).
RING_SHAPES = [(300, 12800, 32), (50, 3200, 16), (4645, 3072, 32)]


@pytest.mark.parametrize("M,K,rank", RING_SHAPES, ids=lambda v: str(v))
def test_act_quant_ring_paths(M, K, rank):
    note(f"act_quant ring M={M} K={K} rank={rank}")
    x = synth.make_matrix_bf16(M, K, seed=K + rank, std=1.5)
    rng = np.random.default_rng(K)
    inv = rng.uniform(0.3, 2.5, K).astype(np.float32)
    l1 = numfmt.f32_to_bf16_bits((rng.standard_normal((K, rank)) * 0.05).astype(np.float32))
    qx, sx, xl1 = lib.quantize_act(dev_u16(x), dev(inv), dev_u16(osv.pack_l1_tiles(l1)), rank)
    torch.cuda.synchronize()
    qa = osv.quantize_act(x, inv, l1)
    check_act(qa, qx, sx, xl1, rank)


def test_act_quant_edge_values():
    """Zero rows, tiny (fp16-subnormal scale) groups, huge groups (saturated
    scale) and exact ties, against the oracle bit for bit."""
    note("act_quant edge values")
    M, K = 20, 256
    rng = np.random.default_rng(8)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[0] = 0.0
    xf[1, :64] = 0.0
    xf[2] *= 1e-6
    xf[3, 64:128] *= 1e-9
    xf[4] *= 3e5
    xf[5] = np.round(xf[5] * 4) / 4          # many exact halves after scaling
    xf[6, :64] = np.arange(64) - 32.0
    xbits = numfmt.f32_to_bf16_bits(xf)
    qx, sx, _ = lib.quantize_act(dev_u16(xbits), None, None, 0)
    torch.cuda.synchronize()
    qa = osv.quantize_act(xbits, None, None)
    check_act(qa, qx, sx, None, 0)


def test_act_quant_empty():
    note("act_quant M=0")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    qx, sx, _ = lib.quantize_act(x, None, None, 0)
    torch.cuda.synchronize()
    assert qx.shape == (0, 64)


def partials_gpu(qx_d, qw_d, M, K, N, m0, mc, n0, nc):
    p = torch.full((mc, nc, K // 64), -12345, dtype=torch.int32, device="cuda")
    lib.svdq_gemm_w4a4_partials(qx_d, M, K, qw_d, N, m0, mc, n0, nc, p)
    torch.cuda.synchronize()
    return p.cpu().numpy()


def test_partials_tiny_all():
    note("partials tiny")
    cfg, li, w = layer("tiny")
    qa = osv.quantize_act(li.x, w.inv_lambda, w.l1)
    M, K, N = cfg.M, cfg.K, cfg.N
    p = partials_gpu(dev(qa.qx), dev(w.qw), M, K, N, 0, M, 0, N)
    assert np.array_equal(p, osv.group_partials(qa.codes, w.qw_codes))


@pytest.mark.parametrize("rect", [(0, 64, 0, 96), (4000, 96, 9100, 116), (1234, 77, 4321, 200),
                                  (2048, 128, 0, 9216)])
def test_partials_qkv_sampled(rect):
    m0, mc, n0, nc = rect
    note(f"partials qkv rect={rect}")
    cfg, li, w = layer("qkv")
    qa = osv.quantize_act(li.x, w.inv_lambda, w.l1)
    p = partials_gpu(dev(qa.qx), dev(w.qw), cfg.M, cfg.K, cfg.N, m0, mc, n0, nc)
    ref = osv.group_partials(qa.codes[m0:m0 + mc], w.qw_codes[n0:n0 + nc])
    assert np.array_equal(p, ref)


def gemm_gpu(qa, dw, rank, act="none", out=torch.bfloat16, bias=True):
    return lib.w4a4_linear(dev(qa.qx), dev_scales(qa.sx), dev(qa.xl1) if rank else None, dw.qw, dw.sw,
                           dw.l2t, dw.bias if bias else None, rank, act=act, out_dtype=out)


@pytest.mark.parametrize("act,bias", [("none", True), ("gelu_tanh", True), ("gelu_tanh", False)])
def test_gemm_tiny(act, bias):
    note(f"gemm tiny act={act} bias={bias}")
    cfg, li, w = layer("tiny")
    dw = DevSvdq(w)
    qa = osv.quantize_act(li.x, w.inv_lambda, w.l1)
    y32 = gemm_gpu(qa, dw, cfg.rank, act, torch.float32, bias)
    ybf = gemm_gpu(qa, dw, cfg.rank, act, torch.bfloat16, bias)
    torch.cuda.synchronize()
    b = w.bias if bias else None
    pre64 = osv.linear_output(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1, w.l2, b)
    y64 = osv.gelu_tanh(pre64) if act == "gelu_tanh" else pre64
    tmag = magnitude_sum(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1, w.l2, b)
    y32h = y32.cpu().numpy()
    if act == "gelu_tanh":
        assert_fp32_gelu(y32h, pre64, fp32_bound(tmag, cfg.K // 64 + cfg.rank))
    else:
        assert_fp32_output(y32h, y64, tmag, cfg.K // 64 + cfg.rank)
    assert_bf16_is_rounded_fp32(host_u16(ybf), y32h)
    assert rel_fro(host_bf16_f64(ybf), y64) <= 2e-3


def test_gemm_ragged_rank0_and_rank128():
    """Ragged M and N against the 128 x 128 tile, rank 0 (plain W4A4), the
    maximum rank, and a rank that ends in a half chunk (32 + 16 ranks); K
    values whose group count is not a multiple of 4 (padded scale quads)."""
    for (M, K, N, r) in [(77, 192, 200, 0), (130, 320, 136, 128), (1, 64, 16, 16), (300, 704, 264, 48)]:
        note(f"gemm ragged M={M} K={K} N={N} r={r}")
        x = synth.make_matrix_bf16(M, K, seed=M, std=1.0)
        wb = synth.make_matrix_bf16(K, N, seed=N, std=0.05)
        b = synth.make_matrix_bf16(1, N, seed=3, std=0.02)[0]
        w = osv.prepare_svdq(x, wb, b, r)
        dw = DevSvdq(w)
        qx, sx, xl1 = lib.quantize_act(dev_u16(x), dw.inv_lambda, dw.l1t, r)
        y = lib.w4a4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, r, out_dtype=torch.float32)
        ybf = lib.w4a4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, r)
        torch.cuda.synchronize()
        qa, y64 = osv.forward(w, x)
        check_act(qa, qx, sx, xl1, r)
        tmag = magnitude_sum(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1 if r else None, w.l2, w.bias)
        assert_fp32_output(y.cpu().numpy(), y64, tmag, K // 64 + r)
        assert_bf16_is_rounded_fp32(host_u16(ybf), y.cpu().numpy())


def test_gemm_empty_and_strided_output():
    note("gemm M=0 and ldy > N")
    cfg, li, w = layer("tiny")
    dw = DevSvdq(w)
    qa = osv.quantize_act(li.x, w.inv_lambda, w.l1)
    y0 = torch.empty((0, cfg.N), dtype=torch.bfloat16, device="cuda")
    lib.svdq_gemm_w4a4(dev(qa.qx), dev_scales(qa.sx), 0, cfg.K, dw.qw, dw.sw, cfg.N, None, None, 0,
                       None, 0, y0, 0, cfg.N)
    big = torch.full((cfg.M, cfg.N + 64), 7.0, dtype=torch.float32, device="cuda")
    lib.svdq_gemm_w4a4(dev(qa.qx), dev_scales(qa.sx), cfg.M, cfg.K, dw.qw, dw.sw, cfg.N, dev(qa.xl1),
                       dw.l2t, cfg.rank, dw.bias, 0, big, 1, cfg.N + 64)
    torch.cuda.synchronize()
    yb = big.cpu().numpy()
    assert np.all(yb[:, cfg.N:] == 7.0)                     # padding untouched
    y64 = osv.linear_output(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1, w.l2, w.bias)
    assert rel_fro(yb[:, :cfg.N], y64) <= 1e-5


def test_qkv_linear_full_size():
    """The QKV workload end to end on the GPU (act + GEMM, the launches the
    benchmark times). Every code and scale is compared; outputs are compared
    on sampled rows, which the oracle computes one row block at a time:
    the GEMM alone on the oracle's operands (element-wise fp32 bound, bf16 =
    RTNE of fp32), and the chained act -> GEMM result (relative bars)."""
    note("qkv linear full size")
    cfg, li, w = layer("qkv")
    dw = DevSvdq(w)
    qx, sx, xl1 = run_act(li.x, dw, cfg.rank)
    y = lib.w4a4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank)
    y2 = lib.w4a4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    qa = osv.quantize_act(li.x, w.inv_lambda, w.l1)
    check_act(qa, qx, sx, xl1, cfg.rank)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(cfg.M - 8, cfg.M),
                                     np.random.default_rng(0).choice(cfg.M, 48, replace=False)]))
    y64 = osv.linear_output(qa.codes[rows], qa.sx[rows], w.qw_codes, w.sw, qa.xl1[rows], w.l2, w.bias)
    # chained GPU path
    assert rel_fro(host_bf16_f64(y)[rows], y64) <= 2e-3
    yf = lib.w4a4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_fro(yf.cpu().numpy()[rows], y64) <= 1e-5
    # GEMM alone on the oracle's operands
    qxo, sxo, xlo = dev(qa.qx), dev_scales(qa.sx), dev(qa.xl1)
    y32 = lib.w4a4_linear(qxo, sxo, xlo, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank, out_dtype=torch.float32)
    ybf = lib.w4a4_linear(qxo, sxo, xlo, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank)
    torch.cuda.synchronize()
    tmag = magnitude_sum(qa.codes[rows], qa.sx[rows], w.qw_codes, w.sw, qa.xl1[rows], w.l2, w.bias)
    y32h = y32.cpu().numpy()
    assert_fp32_output(y32h[rows], y64, tmag, cfg.K // 64 + cfg.rank)
    assert_bf16_is_rounded_fp32(host_u16(ybf), y32h)
    assert rel_fro(host_bf16_f64(ybf)[rows], y64) <= 2e-3


@pytest.mark.parametrize("name,sizes", [("qkv", (3072, 3072, 3072)), ("tiny", (200, 160, 152))])
def test_fused_projection_column_split(name, sizes):
    """A fused [Q | K | V] layer: each projection's weight side (column
    slices of the packed tensors) with the fused layer's activation side
    gives bit-identical columns of the fused output."""
    note(f"fused projection split {name} {sizes}")
    cfg, li, w = layer(name)
    dw = DevSvdq(w)
    qx, sx, xl1 = run_act(li.x, dw, cfg.rank)
    y = lib.w4a4_linear(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, cfg.rank)
    parts = lib.projection_weights(dw.qw, dw.sw, dw.l2t, dw.bias, sizes)
    ys = [lib.w4a4_linear(qx, sx, xl1, q, s, l2, b, cfg.rank) for (q, s, l2, b) in parts]
    torch.cuda.synchronize()
    for view, yp in zip(lib.split_columns(y, sizes), ys):
        assert torch.equal(view.contiguous().view(torch.int16), yp.view(torch.int16))


def test_act_quant_strided_rows():
    """X rows with a leading dimension beyond K (a column window of a wider
    activation, 16-byte aligned): codes, scales and xl1 as for dense rows."""
    note("act_quant ldx > K")
    M, K, r, pad = 70, 320, 32, 64
    xw = synth.make_matrix_bf16(M, K + pad, seed=11, std=1.5)
    x = np.ascontiguousarray(xw[:, 32:32 + K])
    rng = np.random.default_rng(12)
    inv = rng.uniform(0.3, 2.0, K).astype(np.float32)
    l1 = numfmt.f32_to_bf16_bits((rng.standard_normal((K, r)) * 0.1).astype(np.float32))
    xd = dev_u16(xw)[:, 32:32 + K]
    assert xd.stride(0) == K + pad
    qx, sx, xl1 = lib.quantize_act(xd, dev(inv), dev_u16(osv.pack_l1_tiles(l1)), r)
    torch.cuda.synchronize()
    qa = osv.quantize_act(x, inv, l1)
    check_act(qa, qx, sx, xl1, r)


def test_mlp_pair_full_size():
    """The MLP pair at full size (4608 tokens): fc1 3072 -> 12288 with the GELU
    epilogue, then fc2 12288 -> 3072 whose activation pass reads fc1's bf16
    output (fc2's offline preparation is calibrated on that output). Codes and
    scales of both activation passes are compared in full, xl1 and the GEMM
    outputs on sampled rows."""
    note("mlp pair full size")
    c1, c2 = synth.CONFIGS["mlp_fc1"], synth.CONFIGS["mlp_fc2"]
    li1 = synth.make_layer(c1)
    w1 = osv.prepare_svdq(li1.x, li1.w, li1.bias, c1.rank)
    d1 = DevSvdq(w1)
    qx1, sx1, xl1_1 = run_act(li1.x, d1, c1.rank)
    h = lib.w4a4_linear(qx1, sx1, xl1_1, d1.qw, d1.sw, d1.l2t, d1.bias, c1.rank, act="gelu_tanh")
    h32 = lib.w4a4_linear(qx1, sx1, xl1_1, d1.qw, d1.sw, d1.l2t, d1.bias, c1.rank, act="gelu_tanh",
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa1 = osv.quantize_act(li1.x, w1.inv_lambda, w1.l1)
    check_act(qa1, qx1, sx1, xl1_1, c1.rank)
    rows = sample_rows(c1.M, 4, 24, 1)
    pre1 = osv.linear_output(qa1.codes[rows], qa1.sx[rows], w1.qw_codes, w1.sw, qa1.xl1[rows], w1.l2, w1.bias)
    y64_1 = osv.gelu_tanh(pre1)
    tmag1 = magnitude_sum(qa1.codes[rows], qa1.sx[rows], w1.qw_codes, w1.sw, qa1.xl1[rows], w1.l2, w1.bias)
    h32h = h32.cpu().numpy()
    assert_fp32_gelu(h32h[rows], pre1, fp32_bound(tmag1, c1.K // 64 + c1.rank))
    assert_bf16_is_rounded_fp32(host_u16(h), h32h)
    assert rel_fro(host_bf16_f64(h)[rows], y64_1) <= 2e-3
    del h32, h32h

    note("mlp pair fc2 (K 12288)")
    h_bits = host_u16(h)
    li2 = synth.make_layer(c2, M=8)                  # fc2's weights and bias (its x is not used)
    w2 = osv.prepare_svdq(h_bits, li2.w, li2.bias, c2.rank)
    d2 = DevSvdq(w2)
    qx2, sx2, xl1_2 = lib.quantize_act(h, d2.inv_lambda, d2.l1t, c2.rank)
    y2 = lib.w4a4_linear(qx2, sx2, xl1_2, d2.qw, d2.sw, d2.l2t, d2.bias, c2.rank)
    y2f = lib.w4a4_linear(qx2, sx2, xl1_2, d2.qw, d2.sw, d2.l2t, d2.bias, c2.rank, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qa2 = osv.quantize_act(h_bits, w2.inv_lambda, w2.l1)
    check_act(qa2, qx2, sx2, xl1_2, c2.rank)
    y64_2 = osv.linear_output(qa2.codes[rows], qa2.sx[rows], w2.qw_codes, w2.sw, qa2.xl1[rows],
                              w2.l2, w2.bias)
    tmag2 = magnitude_sum(qa2.codes[rows], qa2.sx[rows], w2.qw_codes, w2.sw, qa2.xl1[rows], w2.l2, w2.bias)
    y2fh = y2f.cpu().numpy()
    assert_fp32_output(y2fh[rows], y64_2, tmag2, c2.K // 64 + c2.rank)
    assert_bf16_is_rounded_fp32(host_u16(y2), y2fh)
    assert rel_fro(host_bf16_f64(y2)[rows], y64_2) <= 2e-3
