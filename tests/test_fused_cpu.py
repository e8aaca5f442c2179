"""Fused projections (bit_quantized_diffusion_svdq_amd/fused.py): the column
order, the slicing of every packed weight-side tensor along N, and that a
column slice of the weight side gives the same columns of the output (the
oracle's definition, fp64). CPU only: the helpers index torch tensors."""
import numpy as np
import pytest
import torch

import bit_quantized_diffusion_svdq_amd as lib
from oracle import mxfp4 as omx, svdq as osv


def test_offsets_and_split_views():
    assert lib.column_offsets([3072, 3072, 3072]) == [0, 3072, 6144, 9216]
    y = torch.arange(4 * 40, dtype=torch.float32).reshape(4, 40)
    q, k, v = lib.split_columns(y, [16, 8, 16])
    assert q.shape == (4, 16) and k.shape == (4, 8) and v.shape == (4, 16)
    assert q.data_ptr() == y.data_ptr() and torch.equal(k, y[:, 16:24]) and torch.equal(v, y[:, 24:])
    with pytest.raises(ValueError):
        lib.split_columns(y, [16, 16])             # widths do not cover the output
    with pytest.raises(ValueError):
        lib.column_offsets([12, 28])               # not multiples of 8


def _int4_layer(rng, N, K, r):
    codes = rng.integers(-7, 8, (N, K)).astype(np.int8)
    sw = (rng.uniform(1e-3, 2e-2, (N, K // 64))).astype(np.float16)
    l2 = (rng.standard_normal((r, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bias = (rng.standard_normal(N).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return codes, sw, l2, bias


@pytest.mark.parametrize("K", [192, 320, 1024])       # scale quads full and partly padded
def test_int4_slices_match_packing_of_the_slice(K):
    rng = np.random.default_rng(K)
    N, r = 64, 16
    codes, sw, l2, bias = _int4_layer(rng, N, K, r)
    qw = torch.from_numpy(osv.pack_int4(codes))
    swp = torch.from_numpy(osv.pack_scales(sw).view(np.int16))
    l2t = torch.from_numpy(np.ascontiguousarray(l2.T).view(np.int16))
    b = torch.from_numpy(bias.view(np.int16))
    parts = lib.projection_weights(qw, swp, l2t, b, [24, 8, 32])
    for (n0, n1), (q_s, s_s, l_s, b_s) in zip([(0, 24), (24, 32), (32, 64)], parts):
        assert np.array_equal(q_s.numpy(), osv.pack_int4(codes[n0:n1]))
        assert np.array_equal(s_s.numpy().view(np.uint16), osv.pack_scales(sw[n0:n1]).view(np.uint16))
        assert np.array_equal(l_s.numpy().view(np.uint16), np.ascontiguousarray(l2[:, n0:n1].T))
        assert np.array_equal(b_s.numpy().view(np.uint16), bias[n0:n1])
        assert q_s.is_contiguous() and s_s.is_contiguous()


def test_mxfp4_scale_slices_match_packing_of_the_slice():
    rng = np.random.default_rng(5)
    N, K = 40, 320                                   # 10 blocks: a padded quad
    exps = rng.integers(-20, 5, (N, K // 32)).astype(np.int16)
    codes = rng.integers(-7, 8, (N, K)).astype(np.int8)
    qw = torch.from_numpy(omx.pack_fp4(codes))
    sw = torch.from_numpy(omx.pack_scales(exps))
    q_s, s_s, _, _ = lib.column_slice(qw, sw, None, None, 8, 32)
    assert np.array_equal(q_s.numpy(), omx.pack_fp4(codes[8:32]))
    assert np.array_equal(s_s.numpy(), omx.pack_scales(exps[8:32]))


def test_column_slice_gives_output_columns():
    """With the fused layer's activation side, the weight side of a column
    range gives those output columns (oracle definition, fp64)."""
    rng = np.random.default_rng(9)
    M, K, N, r = 5, 256, 48, 16
    codes, sw, l2, bias = _int4_layer(rng, N, K, r)
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    sx = rng.uniform(1e-2, 1e-1, (M, K // 64)).astype(np.float16)
    xl1 = rng.standard_normal((M, r)).astype(np.float32)
    full = osv.linear_output(qx, sx, codes, sw, xl1, l2, bias)
    for n0, n1 in [(0, 16), (16, 24), (24, 48)]:
        part = osv.linear_output(qx, sx, codes[n0:n1], sw[n0:n1], xl1, l2[:, n0:n1], bias[n0:n1])
        # the library matmul may block differently for a narrower N: fp64 closeness
        np.testing.assert_allclose(part, full[:, n0:n1], rtol=1e-13, atol=0)


def test_column_slice_rejects_bad_ranges():
    qw = torch.zeros((32, 32), dtype=torch.uint8)
    sw = torch.zeros((1, 32, 4), dtype=torch.float16)
    for n0, n1 in [(0, 36), (4, 16), (16, 16), (-8, 8)]:
        with pytest.raises(ValueError):
            lib.column_slice(qw, sw, None, None, n0, n1)
    with pytest.raises(ValueError):
        lib.column_slice(qw, torch.zeros((32, 4), dtype=torch.float16), None, None, 0, 8)


def test_mlp_block_needs_one_format():
    """SvdqMLP runs both layers in one format (the fused epilogue quantises H
    for a next layer of the same format); a mixed pair is refused before any
    buffer is allocated."""
    z = torch.zeros(1)
    fc1 = lib.SvdqLinear(z, None, None, torch.zeros((256, 64), dtype=torch.uint8), z, None, 0, fmt="int4")
    fc2 = lib.SvdqLinear(z, None, None, torch.zeros((64, 128), dtype=torch.uint8), z, None, 0, fmt="mxfp4")
    with pytest.raises(ValueError, match="format"):
        lib.SvdqMLP(fc1, fc2, 64)
    fc3 = lib.SvdqLinear(z, None, None, torch.zeros((64, 128), dtype=torch.uint8), z, None, 0, fmt="nvfp4")
    with pytest.raises(ValueError, match="format"):
        lib.SvdqMLP(fc3, fc3, 64)
