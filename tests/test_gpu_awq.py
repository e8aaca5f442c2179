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
