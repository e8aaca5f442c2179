"""GPU parity of the AWQ W4A16 GEMV against the CPU oracle, through the C ABI."""
import functools

import numpy as np
import pytest
import torch

import synth
from oracle import awq as oawq, numfmt
from gpu_util import assert_bf16_output, dev, dev_f16, dev_u16, host_bf16_f64, note, rel_fro

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib


def run(x_bits, w):
    # the kernel reads codes, scales and zero points in the GEMV tile layout written by
    # the oracle's packer
    return lib.awq_gemv(dev_u16(x_bits), dev(w.inv_s), dev(w.qwt), dev_f16(w.scale_t), dev_f16(w.zero_t),
                        dev_u16(w.bias) if w.bias is not None else None, N=w.N)


def check(y, x_bits, w):
    # fp32 accumulation of x~ (128 + q) before the zero-point fold loses
    # ~7 bits of the 24: allowance 3e-5 * rms on top of the output rounding
    y64 = oawq.gemv(x_bits, w)
    assert_bf16_output(host_bf16_f64(y), y64, 3e-5)


@functools.lru_cache(maxsize=None)
def full_layer():
    cfg = synth.CONFIGS["awq"]
    li = synth.make_layer(cfg)
    return li, oawq.prepare_awq(li.w, li.chan_scale, li.bias)


def test_awq_full_size():
    note("awq gemv full size 4 x 3072 -> 18432")
    li, w = full_layer()
    y = run(li.x, w)
    y2 = run(li.x, w)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    check(y, li.x, w)


# row quads 1, 2 and 4; an odd number of group pairs (uneven K parts); waves
# without pairs (K 128, 256); more pairs per wave than one batch holds (the
# batch loop: 1 row at K 16384 with one tile per workgroup, 4 rows at K 6144
# with five); two LDS chunks (16 rows, K 3072); partial workgroups (N not a
# multiple of 64)
@pytest.mark.parametrize("M,K,N,scaled,bias", [(1, 128, 16, False, False), (16, 256, 48, True, True),
                                               (16, 3072, 80, True, True), (5, 1024, 32, True, True),
                                               (7, 2176, 32, True, False), (3, 8192, 64, True, True),
                                               (2, 3072, 18432 - 64 * 3 + 16, True, True),
                                               (1, 16384, 32, True, True),
                                               (4, 6144, 18432 - 64 * 3 + 16, True, False)])
def test_awq_shapes(M, K, N, scaled, bias):
    note(f"awq gemv M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 1000 + K)
    wb = synth.make_matrix_bf16(K, N, seed=K + N, std=0.02)
    sc = rng.uniform(0.5, 2.0, K).astype(np.float32) if scaled else None
    b = synth.make_matrix_bf16(1, N, seed=1, std=0.02)[0] if bias else None
    w = oawq.prepare_awq(wb, sc, b)
    x = synth.make_matrix_bf16(M, K, seed=M + 7)
    y = run(x, w)
    torch.cuda.synchronize()
    check(y, x, w)



# ---------------------------------------------------------------- weight quantisation on the GPU

@pytest.mark.parametrize("K,N,scaled,strided", [(3072, 18432, True, False), (256, 48, False, False),
                                                (640, 64, True, True), (128, 16, True, False)])
def test_awq_quantize_weight_bit_exact(K, N, scaled, strided):
    """quantize_awq on the GPU gives the oracle's codes, scales and zero
    points in the GEMV tile layouts bit for bit (full adaLN size; no channel
    scale; strided weight rows; one group pair), including groups the test
    makes degenerate: a constant group (range below the 1e-5 floor), an
    all-negative and an all-positive group (zero point clamped at 15 / 0);
    the GEMV on the GPU-quantised weights then equals the GEMV on the
    oracle's arrays bit for bit."""
    note(f"awq quantize weight K={K} N={N} scaled={scaled} strided={strided}")
    rng = np.random.default_rng(K + N)
    wb = synth.make_matrix_bf16(K, N, seed=K * 3 + N, std=0.02)
    w64 = numfmt.bf16_bits_to_f32(wb).astype(np.float64)
    w64[0:64, 1] = 0.0125                        # constant group
    w64[64:128, 2] = -np.abs(w64[64:128, 2]) - 0.01   # all negative
    w64[0:64, 3] = np.abs(w64[0:64, 3]) + 0.01        # all positive
    wb = synth.bf16_round(w64.astype(np.float32))
    sc = rng.uniform(0.5, 2.0, K).astype(np.float32) if scaled else None
    ref = oawq.prepare_awq(wb, sc)
    wt = dev_u16(wb)
    if strided:
        big = torch.zeros((K, N + 24), dtype=torch.bfloat16, device="cuda")
        big[:, :N] = wt
        wt = big[:, :N]
    out = lib.quantize_awq(wt, dev(ref.inv_s) if scaled else None)
    torch.cuda.synchronize()
    assert np.array_equal(out["qwt"].cpu().numpy(), ref.qwt)
    assert np.array_equal(out["scale_t"].cpu().numpy().view(np.uint16), np.asarray(ref.scale_t, np.float16).view(np.uint16))
    assert np.array_equal(out["zero_t"].cpu().numpy().view(np.uint16), np.asarray(ref.zero_t, np.float16).view(np.uint16))
    x = synth.make_matrix_bf16(4, K, seed=K + 1)
    inv = dev(ref.inv_s)
    y_gpu = lib.awq_gemv(dev_u16(x), inv, out["qwt"], out["scale_t"], out["zero_t"], None, N=N)
    y_ref = lib.awq_gemv(dev_u16(x), inv, dev(ref.qwt), dev_f16(ref.scale_t), dev_f16(ref.zero_t), None, N=N)
    torch.cuda.synchronize()
    assert torch.equal(y_gpu.view(torch.int16), y_ref.view(torch.int16))


def test_awq_packaged_layer_round_trip(tmp_path):
    """quantize_awq on the GPU, save_awq_layer, load_awq_layer: the loaded
    arrays are the quantiser's byte for byte and the GEMV gives bit-identical
    outputs."""
    K, N = 512, 64
    note(f"awq packaged layer K={K} N={N}")
    wb = synth.make_matrix_bf16(K, N, seed=11, std=0.02)
    sc = np.random.default_rng(12).uniform(0.5, 2.0, K).astype(np.float32)
    inv = dev((1.0 / sc.astype(np.float64)).astype(np.float32))
    b = dev_u16(synth.make_matrix_bf16(1, N, seed=13, std=0.02)[0])
    out = lib.quantize_awq(dev_u16(wb), inv)
    p = str(tmp_path / "awq.safetensors")
    lib.save_awq_layer(p, out, bias=b)
    back = lib.load_awq_layer(p, device="cuda")
    for name in ("qwt", "scale_t", "zero_t", "inv_s"):
        assert torch.equal(out[name].view(torch.uint8), back[name].view(torch.uint8)), name
    x = dev_u16(synth.make_matrix_bf16(3, K, seed=14))
    ya = lib.awq_gemv(x, out["inv_s"], out["qwt"], out["scale_t"], out["zero_t"], b, N=N)
    yb = lib.awq_gemv(x, back["inv_s"], back["qwt"], back["scale_t"], back["zero_t"], back["bias"], N=N)
    yc = lib.awq_linear(x, back)                            # the dict's own bias
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    assert torch.equal(ya.view(torch.int16), yc.view(torch.int16))
