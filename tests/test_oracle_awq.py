"""Pins for the oracle's AWQ W4A16 GEMV."""
import os

import numpy as np
import pytest

import synth
from oracle import awq, numfmt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    d = {}
    for line in open(os.path.join(GOLDEN, "awq_group.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        d[k] = v
    return d


def test_qasym64_golden():
    d = _golden()
    v = np.full(64, 0.25, np.float32)
    v[:16] = np.array([i * 0.1 - 0.5 for i in range(16)], np.float64).astype(np.float32)
    s, z, q = awq.qasym64(v[None, :])
    assert numfmt.f16_bits(s)[0] == int(d["scale"][0], 16)
    assert float(z[0]) == float(d["zero"][0])
    assert list(q[0, :16]) == [int(t) for t in d["codes_head"]]
    assert np.all(q[0, 16:] == int(d["codes_tail"][0]))


def test_qasym64_bounds():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((3000, 64)) * np.exp(rng.uniform(-6, 3, (3000, 1)))).astype(np.float32)
    v[:100] += 5.0             # groups entirely positive: zero point clips at 0
    s, z, q = awq.qasym64(v)
    sf = s.astype(np.float64)
    deq = (q.astype(np.float64) - z.astype(np.float64)[:, None]) * sf[:, None]
    err = np.abs(deq - v)
    clipped = (q == 0) | (q == 15)
    assert np.all(err[~clipped] <= (sf / 2 * (1 + 2.0 ** -9))[:, None].repeat(64, 1)[~clipped])
    assert np.all(z >= 0) and np.all(z <= 15) and q.max() <= 15
    assert np.array_equal(z.astype(np.float64), np.round(z.astype(np.float64)))


def test_pack_u4_roundtrip():
    c = np.arange(32, dtype=np.uint8).reshape(2, 16) % 16
    p = awq.pack_u4(c)
    assert p[0, 0] == 0x10 and p[0, 1] == 0x32
    assert np.array_equal(awq.unpack_u4(p), c)


def _brute(x_bits, wts):
    x = numfmt.bf16_bits_to_f32(x_bits)
    M = x.shape[0]
    y = np.zeros((M, wts.N))
    for m in range(M):
        for n in range(wts.N):
            acc = 0.0
            for k in range(wts.K):
                g = k // 64
                xs = float(np.float32(x[m, k] * wts.inv_s[k]))
                acc += xs * (int(wts.codes[n, k]) - float(wts.zero[n, g])) * float(wts.scale[n, g])
            y[m, n] = acc + float(numfmt.bf16_bits_to_f32(wts.bias)[n])
    return y


def test_gemv_brute_force_tiny():
    rng = np.random.default_rng(1)
    K, N, M = 128, 6, 3
    w = numfmt.f32_to_bf16_bits((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    sc = rng.uniform(0.5, 2.0, K).astype(np.float32)
    b = numfmt.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32) * 0.02)
    wts = awq.prepare_awq(w, sc, b)
    x = synth.make_matrix_bf16(M, K, seed=2)
    y = awq.gemv(x, wts)
    assert np.allclose(y, _brute(x, wts), rtol=1e-12, atol=1e-14)


def test_gemv_grid_exact_and_unit_channel_scale():
    """Weights already on an asymmetric 4-bit grid with power-of-two steps and
    s_c = 1: quantisation is lossless and the GEMV equals x @ W + bias."""
    rng = np.random.default_rng(2)
    K, N, M = 192, 16, 4
    q = rng.integers(0, 16, (K, N)).astype(np.float64)
    q[0::64] = 0
    q[1::64] = 15                      # every group spans the full 0..15 range
    z = rng.integers(0, 16, (K // 64, N)).astype(np.float64)
    step = 2.0 ** rng.integers(-9, -5, (K // 64, N))
    w = ((q - np.repeat(z, 64, axis=0)) * np.repeat(step, 64, axis=0)).astype(np.float32)
    w_bits = numfmt.f32_to_bf16_bits(w)
    assert np.array_equal(numfmt.bf16_bits_to_f32(w_bits), w)
    wts = awq.prepare_awq(w_bits, None)
    wts1 = awq.prepare_awq(w_bits, np.ones(K, np.float32))
    assert np.array_equal(wts.qw, wts1.qw) and np.array_equal(wts.scale, wts1.scale)
    assert np.array_equal(wts.scale.astype(np.float64), step.T)
    x = synth.make_matrix_bf16(M, K, seed=3)
    ref = numfmt.bf16_bits_to_f32(x).astype(np.float64) @ w.astype(np.float64)
    assert np.allclose(awq.gemv(x, wts), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_channel_scale_moves_into_weight():
    """x * inv_s times W / inv_s: with weights on the grid after scaling, the
    output equals x @ W (the activation-aware scale changes nothing exact)."""
    rng = np.random.default_rng(3)
    K, N = 128, 8
    sc = (2.0 ** rng.integers(-1, 2, K)).astype(np.float32)   # powers of two: exact
    q = rng.integers(0, 16, (K, N)).astype(np.float64)
    q[0::64] = 0
    q[1::64] = 15
    w_scaled = (q - 8) * 2.0 ** -7                              # W' on the grid
    w = (w_scaled / sc[:, None].astype(np.float64)).astype(np.float32)
    wts = awq.prepare_awq(numfmt.f32_to_bf16_bits(w), sc)
    x = synth.make_matrix_bf16(2, K, seed=4)
    ref = numfmt.bf16_bits_to_f32(x).astype(np.float64) @ w.astype(np.float64)
    assert np.allclose(awq.gemv(x, wts), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_tile_layout_spot_checks():
    """The GEMV tile layout [N/16][K/128][16][64]: flat offset of block
    (t, j, c), byte b is ((t * K/128 + j) * 16 + c) * 64 + b, and it holds byte
    64 j + b of plain row 16 t + c. Each plain byte is made unique so a wrong
    index shows; offsets below are worked out by hand for N = 32, K = 256."""
    N, K = 32, 256
    plain = np.arange(N * K // 2, dtype=np.int64).reshape(N, K // 2)
    plain = (plain * 7 + plain // 251) % 256          # distinct neighbours, all bytes used
    plain = plain.astype(np.uint8)
    flat = awq.tile_for_gemv(plain)
    assert flat.shape == (N * K // 2,)
    # (t=0, j=0, c=0, b=0) -> offset 0, plain[0][0]
    assert flat[0] == plain[0, 0]
    # (t=0, j=0, c=1, b=0) -> offset 64, plain[1][0]
    assert flat[64] == plain[1, 0]
    # (t=0, j=1, c=0, b=0) -> offset (1 * 16) * 64 = 1024, plain[0][64]
    assert flat[1024] == plain[0, 64]
    # (t=1, j=1, c=3, b=5) -> ((1 * 2 + 1) * 16 + 3) * 64 + 5 = 3269, plain[19][69]
    assert flat[3269] == plain[19, 69]
    # last byte: (t=1, j=1, c=15, b=63) -> 4095, plain[31][127]
    assert flat[4095] == plain[31, 127]
    # a permutation: every plain byte appears exactly once
    assert np.array_equal(np.sort(flat), np.sort(plain.ravel()))


def test_tile_layout_rejects_ragged():
    with pytest.raises(ValueError):
        awq.tile_for_gemv(np.zeros((24, 64), np.uint8))
    with pytest.raises(ValueError):
        awq.tile_for_gemv(np.zeros((16, 96), np.uint8))


def test_tile_scales_spot_checks():
    """[N/16][G][16]: flat offset of (t, g, c) is (t * G + g) * 16 + c and holds
    a[16 t + c, g]; offsets worked out by hand for N = 32, G = 3."""
    a = (np.arange(32 * 3).reshape(32, 3) * 5 % 97).astype(np.float16)
    f = awq.tile_scales_for_gemv(a)
    assert f[0] == a[0, 0]                 # (0, 0, 0)
    assert f[1] == a[1, 0]                 # (0, 0, 1)
    assert f[16] == a[0, 1]                # (0, 1, 0)
    assert f[(1 * 3 + 2) * 16 + 7] == a[23, 2]   # (1, 2, 7) -> 87
    assert f[95] == a[31, 2]
    assert np.array_equal(np.sort(f), np.sort(a.ravel()))
