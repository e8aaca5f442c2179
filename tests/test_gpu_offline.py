"""GPU offline quantiser against the oracle's offline steps (calibration,
smoothing, low-rank branch, residual quantisation and packing).

Bars: calibration maxima, inv_lambda (alpha 0.5), W_hat, codes and scales
bit-exact; the truncated SVD from the same random test matrix gives the
same singular values to 1e-9 (relative) and the same bf16 factors except
where an fp64 value lies within rounding noise of a bf16 rounding boundary
(then one ulp apart, and rare). Codes and scales are checked bit-exact
given the same factors: the oracle's factors, and the GPU's own."""
import numpy as np
import pytest
import torch

import synth
from oracle import linalg as olin
from oracle import mxfp4 as omx
from oracle import svdq as osv
from oracle.numfmt import bf16_bits_to_f32
from gpu_util import dev, dev_u16, host_u16, note, rel_fro

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib


def _f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def _layer(name, M=None):
    li = synth.make_layer(synth.CONFIGS[name], M=M)
    return li, bf16_bits_to_f32(li.x), bf16_bits_to_f32(li.w)


# ---------------------------------------------------------------- calibration

@pytest.mark.parametrize("rows,cols", [(333, 320), (1, 8), (4096, 3072)])
def test_calib_absmax_bit_exact(rows, cols):
    note(f"offline calib absmax {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    a = rng.standard_normal((rows, cols)).astype(np.float32) * rng.uniform(0.1, 10.0, cols).astype(np.float32)
    a[rng.integers(0, rows, 5), rng.integers(0, cols, 5)] = -1e3          # negative extremes
    bits = synth.bf16_round(a)
    af = bf16_bits_to_f32(bits)
    ax_ref, aw_ref = osv.calib_absmax(af, af)                             # max over rows, over columns
    d = dev_u16(bits)
    ax = torch.empty(cols, dtype=torch.float32, device="cuda")
    aw = torch.full((rows,), 7.0, dtype=torch.float32, device="cuda")    # overwritten (accumulate 0)
    lib.svdq_calib_absmax(d, rows, cols, cols, 0, 0, ax)
    lib.svdq_calib_absmax(d, rows, cols, cols, 1, 0, aw)
    assert np.array_equal(_f32_bits(ax), ax_ref.view(np.uint32))
    assert np.array_equal(_f32_bits(aw), aw_ref.view(np.uint32))


def test_calib_absmax_accumulates_batches_and_strides():
    note("offline calib absmax over batches, strided rows")
    rng = np.random.default_rng(3)
    b1 = synth.bf16_round(rng.standard_normal((200, 264)).astype(np.float32))
    b2 = synth.bf16_round((rng.standard_normal((77, 264)) * 3).astype(np.float32))
    ref, _ = osv.calib_absmax(bf16_bits_to_f32(np.concatenate([b1, b2])), np.zeros((264, 1), np.float32))
    pad = np.zeros((77, 272), np.uint16)
    pad[:, :264] = b2
    ax = torch.empty(264, dtype=torch.float32, device="cuda")
    lib.svdq_calib_absmax(dev_u16(b1), 200, 264, 264, 0, 0, ax)
    lib.svdq_calib_absmax(dev_u16(pad), 77, 264, 272, 0, 1, ax)          # ld 272 > cols, folded in
    assert np.array_equal(_f32_bits(ax), ref.view(np.uint32))


# ---------------------------------------------------------------- smoothing

def _stats(K, seed):
    rng = np.random.default_rng(seed)
    ax = rng.uniform(1e-3, 60.0, K).astype(np.float32)
    aw = rng.uniform(1e-4, 0.2, K).astype(np.float32)
    ax[::37] = 0.0
    aw[5::41] = 0.0
    return ax, aw


@pytest.mark.parametrize("alpha", [0.5, 0.0, 1.0])
def test_smoothing_bit_exact(alpha):
    note(f"offline smoothing alpha {alpha}")
    ax, aw = _stats(3072, 11)
    _, inv_ref = osv.smoothing(ax, aw, alpha)
    inv = torch.empty(3072, dtype=torch.float32, device="cuda")
    lib.svdq_smoothing(dev(ax), dev(aw), 3072, alpha, inv)
    assert np.array_equal(_f32_bits(inv), inv_ref.view(np.uint32))


def test_smoothing_general_alpha_within_an_ulp():
    """Other exponents go through pow on both sides; libm and the device's
    pow may differ in the last fp64 bit, which can move inv_lambda by one
    fp32 ulp only where it sits on a rounding boundary."""
    note("offline smoothing alpha 0.3")
    ax, aw = _stats(4096, 12)
    _, inv_ref = osv.smoothing(ax, aw, 0.3)
    inv = torch.empty(4096, dtype=torch.float32, device="cuda")
    lib.svdq_smoothing(dev(ax), dev(aw), 4096, 0.3, inv)
    d = np.abs(_f32_bits(inv).astype(np.int64) - inv_ref.view(np.uint32).astype(np.int64))
    assert d.max() <= 1 and np.count_nonzero(d) <= 4


def test_smooth_weight_bit_exact():
    note("offline smooth weight 512 x 520")
    rng = np.random.default_rng(4)
    w = synth.bf16_round((rng.standard_normal((512, 520)) * 0.02).astype(np.float32))
    inv = rng.uniform(0.05, 3.0, 512).astype(np.float32)
    ref = osv.smooth_weight(bf16_bits_to_f32(w), inv)
    wpad = np.zeros((512, 528), np.uint16)
    wpad[:, :520] = w
    out = torch.empty((512, 520), dtype=torch.float64, device="cuda")
    lib.svdq_smooth_weight(dev_u16(wpad), 512, 520, 528, dev(inv), out)
    assert np.array_equal(out.cpu().numpy().view(np.uint64), ref.view(np.uint64))
    out1 = torch.empty((512, 520), dtype=torch.float64, device="cuda")
    lib.svdq_smooth_weight(dev_u16(w), 512, 520, 520, None, out1)        # inv_lambda NULL = 1
    assert np.array_equal(out1.cpu().numpy(), bf16_bits_to_f32(w).astype(np.float64))


# ---------------------------------------------------------------- low-rank branch

def _gpu_lowrank(w_hat, rank, omega, iters=4):
    K, N = w_hat.shape
    l = omega.shape[1]
    nbytes = lib.svdq_lowrank_workspace_size(K, N, rank, l)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    l1 = torch.empty((K, rank), dtype=torch.bfloat16, device="cuda")
    l2 = torch.empty((rank, N), dtype=torch.bfloat16, device="cuda")
    sig = torch.empty(rank, dtype=torch.float64, device="cuda")
    lib.svdq_lowrank(dev(w_hat), K, N, rank, dev(omega), l, iters, l1, l2, sig, ws, nbytes)
    return host_u16(l1), host_u16(l2), sig.cpu().numpy()


def _bf16_close(a_bits, b_bits):
    """(fraction of entries that differ, largest difference in bf16 ulps)"""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    d = np.abs(a - b)
    return np.count_nonzero(d) / d.size, int(d.max(initial=0))


@pytest.mark.parametrize("name,M", [("tiny", None), ("qkv", 512)])
def test_lowrank_matches_oracle(name, M):
    li, x, w = _layer(name, M)
    cfg = li.cfg
    note(f"offline lowrank {name} K={cfg.K} N={cfg.N} r={cfg.rank}")
    ax, aw = osv.calib_absmax(x, w)
    _, inv = osv.smoothing(ax, aw, cfg.alpha)
    w_hat = osv.smooth_weight(w, inv)
    l = min(cfg.rank + 16, min(w_hat.shape))
    omega = np.random.default_rng(0).standard_normal((cfg.N, l))
    u, s, vt = olin.randomized_svd(w_hat, cfg.rank, omega, power_iters=4)
    l1_ref = osv.f64_to_bf16_bits(u * s[None, :])
    l2_ref = osv.f64_to_bf16_bits(vt)
    l1, l2, sig = _gpu_lowrank(w_hat, cfg.rank, omega)
    assert np.max(np.abs(sig - s) / s) < 1e-9
    for got, ref in ((l1, l1_ref), (l2, l2_ref)):
        frac, ulps = _bf16_close(got, ref)
        assert frac <= 1e-4 and ulps <= 1, (frac, ulps)
    # the rank-r approximation itself (Eckart-Young): the error the oracle's
    # factors leave and the GPU's leave are the same
    def err(a, b):
        return np.linalg.norm(w_hat - bf16_bits_to_f32(a).astype(np.float64) @ bf16_bits_to_f32(b).astype(np.float64))
    assert abs(err(l1, l2) - err(l1_ref, l2_ref)) <= 1e-6 * np.linalg.norm(w_hat)


def test_lowrank_exact_when_block_covers_the_matrix():
    """l = min(K, N): the range is the whole column space, so the result is
    the exact truncated SVD (checked against LAPACK's singular values and
    the Eckart-Young error)."""
    note("offline lowrank full block 64 x 200")
    rng = np.random.default_rng(8)
    w_hat = rng.standard_normal((64, 200)) * np.linspace(3.0, 0.01, 64)[:, None]
    omega = rng.standard_normal((200, 64))
    l1, l2, sig = _gpu_lowrank(w_hat, 48, omega, iters=1)
    s_ref = np.linalg.svd(w_hat, compute_uv=False)
    assert np.max(np.abs(sig - s_ref[:48]) / s_ref[:48]) < 1e-9
    approx = bf16_bits_to_f32(l1).astype(np.float64) @ bf16_bits_to_f32(l2).astype(np.float64)
    tail = np.sqrt(np.sum(s_ref[48:] ** 2))
    assert np.linalg.norm(w_hat - approx) <= tail + 1e-2 * np.linalg.norm(w_hat)


# ---------------------------------------------------------------- residual and packing

def _gpu_residual(w_hat, l1, l2, rank):
    K, N = w_hat.shape
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.empty(((K // 64 + 3) // 4, N, 4), dtype=torch.float16, device="cuda")
    lib.svdq_quantize_residual(dev(w_hat), K, N, dev_u16(l1) if rank else None, dev_u16(l2) if rank else None,
                               rank, qw, sw)
    return qw.cpu().numpy(), sw.cpu().numpy()


def _oracle_residual(w_hat, l1, l2, rank):
    K, N = w_hat.shape
    if rank:
        r = osv.residual(w_hat, l1, l2)
    else:
        r = w_hat.astype(np.float32)
    codes, s = osv.quantize_rows(np.ascontiguousarray(r.T))
    return osv.pack_int4(codes), osv.pack_scales(s)


@pytest.mark.parametrize("K,N,rank", [(512, 512, 16), (192, 200, 32), (320, 8, 0), (256, 264, 112), (3072, 9216, 32)])
def test_residual_codes_bit_exact_given_factors(K, N, rank):
    note(f"offline residual K={K} N={N} r={rank}")
    rng = np.random.default_rng(K + N + rank)
    w_hat = rng.standard_normal((K, N)) * 0.03 * rng.uniform(0.2, 5.0, K)[:, None]
    w_hat[:, 3 % N] = 0.0                                  # an all-zero column: scale 0, codes 0
    l1 = synth.bf16_round((rng.standard_normal((K, rank)) * 0.05).astype(np.float32)) if rank else None
    l2 = synth.bf16_round((rng.standard_normal((rank, N)) * 0.05).astype(np.float32)) if rank else None
    if rank:
        w_hat[:, 3 % N] = (bf16_bits_to_f32(l1).astype(np.float64) @ bf16_bits_to_f32(l2).astype(np.float64))[:, 3 % N]
    qw, sw = _gpu_residual(w_hat, l1, l2, rank)
    qw_ref, sw_ref = _oracle_residual(w_hat, l1, l2, rank)
    assert np.array_equal(qw, qw_ref)
    assert np.array_equal(sw.view(np.uint16), sw_ref.view(np.uint16))


def _gpu_residual_mx(w_hat, l1, l2, rank):
    K, N = w_hat.shape
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    # filled with a pattern: the padding of the last record must be written too
    se = torch.full(((K // 64 + 3) // 4, N, 8), 0xAB, dtype=torch.uint8, device="cuda")
    lib.svdq_quantize_residual_mxfp4(dev(w_hat), K, N, dev_u16(l1) if rank else None, dev_u16(l2) if rank else None,
                                     rank, qw, se)
    return qw.cpu().numpy(), se.cpu().numpy()


def _oracle_residual_mx(w_hat, l1, l2, rank):
    r = osv.residual(w_hat, l1, l2) if rank else w_hat.astype(np.float32)
    codes, exps = omx.quantize_rows(np.ascontiguousarray(r.T))
    return omx.pack_fp4(codes), omx.pack_scales(exps)


@pytest.mark.parametrize("K,N,rank", [(512, 512, 16), (192, 200, 32), (320, 8, 0), (256, 264, 112), (3072, 9216, 32)])
def test_residual_mxfp4_bit_exact_given_factors(K, N, rank):
    """The MXFP4 residual quantisation: E2M1 codes and E8M0 exponent records
    bit-exact against the oracle's per-column MXFP4 quantisation of the same
    residual (ragged N, K not a multiple of 256 (padded records), rank 0 and
    112, an all-zero column (exponent -127, codes 0), and at rank 0 a column
    of fp32-subnormal values (clamped exponent)."""
    note(f"offline residual mxfp4 K={K} N={N} r={rank}")
    rng = np.random.default_rng(K + N + rank + 1)
    w_hat = rng.standard_normal((K, N)) * 0.03 * rng.uniform(0.2, 5.0, K)[:, None]
    w_hat[:, 3 % N] = 0.0
    l1 = synth.bf16_round((rng.standard_normal((K, rank)) * 0.05).astype(np.float32)) if rank else None
    l2 = synth.bf16_round((rng.standard_normal((rank, N)) * 0.05).astype(np.float32)) if rank else None
    if rank:
        w_hat[:, 3 % N] = (bf16_bits_to_f32(l1).astype(np.float64) @ bf16_bits_to_f32(l2).astype(np.float64))[:, 3 % N]
    else:
        w_hat[:, 5 % N] *= 1e-38
    qw, se = _gpu_residual_mx(w_hat, l1, l2, rank)
    qw_ref, se_ref = _oracle_residual_mx(w_hat, l1, l2, rank)
    assert np.array_equal(qw, qw_ref)
    assert np.array_equal(se, se_ref)


def test_quantize_layer_mxfp4_end_to_end():
    """quantize_layer(fmt="mxfp4") on the tiny layer: smoothing and factors as
    the INT4 form, the residual in MXFP4 exactly as the oracle quantises the
    GPU's own factors; the MXFP4 online path on the quantised layer matches the
    oracle's MXFP4 forward on the same arrays."""
    li, x, w = _layer("tiny", None)
    cfg = li.cfg
    note(f"offline quantize_layer mxfp4 tiny K={cfg.K} N={cfg.N} r={cfg.rank}")
    out = lib.quantize_layer(dev_u16(li.w), dev_u16(li.x), cfg.rank, alpha=cfg.alpha, bias=dev_u16(li.bias),
                             keep_factors=True, fmt="mxfp4")
    torch.cuda.synchronize()
    l1, l2 = host_u16(out["l1"]), host_u16(out["l2"])
    w_hat = out["w_hat"].cpu().numpy()
    qw_ref, se_ref = _oracle_residual_mx(w_hat, l1, l2, cfg.rank)
    assert out["fmt"] == "mxfp4"
    assert np.array_equal(out["qw"].cpu().numpy(), qw_ref)
    assert np.array_equal(out["sw"].cpu().numpy(), se_ref)
    layer = lib.SvdqLinear.from_quantized(out)
    assert layer.fmt == "mxfp4"
    xs = li.x[:64]
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(xs), layer.inv_lambda, layer.l1t, cfg.rank)
    y = lib.mxfp4_linear(qx, sx, xl1, layer.qw, layer.sw, layer.l2t, layer.bias, cfg.rank,
                         out_dtype=torch.float32).cpu().numpy()
    codes = omx.unpack_fp4(qw_ref)
    exps = omx.unpack_scales(se_ref, cfg.K // 32)
    inv = out["inv_lambda"].cpu().numpy()
    mw = omx.MxWeights(cfg.K, cfg.N, cfg.rank, inv, l1, l2, codes, exps, li.bias)
    _, y64 = omx.forward(mw, xs)
    assert rel_fro(y, y64) < 1e-5


@pytest.mark.parametrize("K,N,rank", [(512, 512, 16), (3072, 9216, 32), (192, 24, 48)])
def test_pack_lowrank_layouts(K, N, rank):
    note(f"offline pack lowrank K={K} N={N} r={rank}")
    rng = np.random.default_rng(K * 3 + rank)
    l1 = synth.bf16_round(rng.standard_normal((K, rank)).astype(np.float32))
    l2 = synth.bf16_round(rng.standard_normal((rank, N)).astype(np.float32))
    l1t = torch.empty(K * rank, dtype=torch.bfloat16, device="cuda")
    l2t = torch.empty((N, rank), dtype=torch.bfloat16, device="cuda")
    lib.svdq_pack_lowrank(dev_u16(l1), dev_u16(l2), K, N, rank, l1t, l2t)
    assert np.array_equal(host_u16(l1t), osv.pack_l1_tiles(l1))
    assert np.array_equal(host_u16(l2t), np.ascontiguousarray(l2.T))


# ---------------------------------------------------------------- whole layer

@pytest.mark.parametrize("name,M", [("tiny", None), ("qkv", 512)])
def test_quantize_layer_end_to_end(name, M):
    """The GPU quantiser on a layer's weight and calibration batch: its
    arrays equal the oracle's prepare (inv_lambda exactly; codes and scales
    exactly given the GPU's own factors; factors as in the low-rank test);
    the online path then runs on them and matches the oracle's forward on
    the same arrays, and the method's error against the exact layer is the
    oracle's."""
    li, x, w = _layer(name, M)
    cfg = li.cfg
    note(f"offline quantize_layer {name} K={cfg.K} N={cfg.N} r={cfg.rank}")
    ref = osv.prepare_svdq(li.x, li.w, li.bias, cfg.rank, alpha=cfg.alpha, keep_w_hat=True)
    out = lib.quantize_layer(dev_u16(li.w), dev_u16(li.x), cfg.rank, alpha=cfg.alpha, bias=dev_u16(li.bias),
                             keep_factors=True)
    torch.cuda.synchronize()
    assert np.array_equal(_f32_bits(out["inv_lambda"]), ref.inv_lambda.view(np.uint32))
    assert np.array_equal(out["w_hat"].cpu().numpy().view(np.uint64), ref.w_hat.view(np.uint64))
    assert np.max(np.abs(out["sigma"].cpu().numpy() - ref.sigma) / ref.sigma) < 1e-9
    l1, l2 = host_u16(out["l1"]), host_u16(out["l2"])
    for got, want in ((l1, ref.l1), (l2, ref.l2)):
        frac, ulps = _bf16_close(got, want)
        assert frac <= 1e-4 and ulps <= 1, (frac, ulps)
    # codes and scales: exactly the oracle's residual quantisation of the
    # GPU's own factors
    qw_ref, sw_ref = _oracle_residual(ref.w_hat, l1, l2, cfg.rank)
    assert np.array_equal(out["qw"].cpu().numpy(), qw_ref)
    assert np.array_equal(out["sw"].cpu().numpy().view(np.uint16), sw_ref.view(np.uint16))
    assert np.array_equal(host_u16(out["l1t"]), osv.pack_l1_tiles(l1))
    assert np.array_equal(host_u16(out["l2t"]), np.ascontiguousarray(l2.T))
    # online path on the GPU-quantised layer: 64 rows
    xs = li.x[:64]
    qx, sx, xl1 = lib.quantize_act(dev_u16(xs), out["inv_lambda"], out["l1t"], cfg.rank)
    y = lib.w4a4_linear(qx, sx, xl1, out["qw"], out["sw"], out["l2t"], out["bias"], cfg.rank,
                        out_dtype=torch.float32).cpu().numpy()
    codes = osv.unpack_int4(qw_ref)
    sw_rows = osv.unpack_scales(sw_ref, cfg.K // 64)
    gw = osv.SvdqWeights(cfg.K, cfg.N, cfg.rank, ref.inv_lambda, l1, l2, codes, qw_ref, sw_rows, li.bias, ref.sigma)
    _, y64 = osv.forward(gw, xs)
    assert rel_fro(y, y64) < 1e-5
    exact = osv.exact_output(xs, li.w, li.bias)
    _, y64_ref = osv.forward(ref, xs)
    e_gpu, e_ref = rel_fro(y, exact), rel_fro(y64_ref, exact)
    assert abs(e_gpu - e_ref) <= 0.02 * e_ref, (e_gpu, e_ref)


def test_packaged_layer_round_trip(tmp_path):
    """Quantize on the GPU, package (save_layer), load back (load_layer): the
    loaded layer's arrays are the quantiser's, byte for byte, and the online
    path on it gives bit-identical outputs."""
    li, x, w = _layer("tiny", None)
    cfg = li.cfg
    note(f"packaged layer tiny K={cfg.K} N={cfg.N} r={cfg.rank}")
    out = lib.quantize_layer(dev_u16(li.w), dev_u16(li.x), cfg.rank, alpha=cfg.alpha, bias=dev_u16(li.bias))
    layer = lib.SvdqLinear.from_quantized(out)
    p = str(tmp_path / "tiny.safetensors")
    lib.save_layer(p, layer, alpha=cfg.alpha, seed=0)
    back = lib.load_layer(p, device="cuda")
    for name in ("inv_lambda", "l1t", "l2t", "qw", "sw", "bias"):
        a, b = getattr(layer, name), getattr(back, name)
        assert b.device.type == "cuda" and a.dtype == b.dtype
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name
    xs = dev_u16(li.x[:64])
    ys = []
    for l in (layer, back):
        qx, sx, xl1 = lib.quantize_act(xs, l.inv_lambda, l.l1t, l.rank)
        ys.append(lib.w4a4_linear(qx, sx, xl1, l.qw, l.sw, l.l2t, l.bias, l.rank))
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


@pytest.mark.parametrize("fmt,act", [("int4", "none"), ("mxfp4", "gelu_tanh")])
def test_layer_call_matches_explicit_launches(fmt, act):
    """SvdqLinear(x) runs the activation pass and the GEMM of its format:
    outputs bit-identical to the two explicit calls, bf16 and fp32, on a
    strided row view."""
    li, x, w = _layer("tiny", None)
    cfg = li.cfg
    note(f"layer call {fmt} act={act}")
    layer = lib.SvdqLinear.from_quantized(
        lib.quantize_layer(dev_u16(li.w), dev_u16(li.x), cfg.rank, alpha=cfg.alpha, bias=dev_u16(li.bias), fmt=fmt))
    big = dev_u16(np.concatenate([li.x[:77], li.x[:77]], axis=1))
    xs = big[:, :cfg.K]                                   # ldx = 2K
    qa = lib.quantize_act if fmt == "int4" else lib.quantize_act_mxfp4
    lin = lib.w4a4_linear if fmt == "int4" else lib.mxfp4_linear
    for dt in (torch.bfloat16, torch.float32):
        y = layer(xs, act=act, out_dtype=dt)
        qx, sx, xl1 = qa(xs, layer.inv_lambda, layer.l1t, layer.rank)
        y_ref = lin(qx, sx, xl1, layer.qw, layer.sw, layer.l2t, layer.bias, layer.rank, act=act, out_dtype=dt)
        torch.cuda.synchronize()
        assert y.dtype == dt and y.shape == (77, cfg.N)
        assert torch.equal(y.view(torch.uint8), y_ref.view(torch.uint8))
