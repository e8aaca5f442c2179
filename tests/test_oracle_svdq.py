"""Pins for the oracle's SVDQuant W4A4 path.

Each test ties the oracle to something other than its own formulas: the
hand-derived fixtures in tests/golden, closed forms, invariants, brute-force
loops on tiny inputs, or plain matrix products of values placed exactly on
the quantisation grid."""
import math
import os

import numpy as np
import pytest

import synth
from oracle import numfmt, svdq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_qsym_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "qsym64_cases.txt")):
        line = line.strip()
        if not line.startswith("case "):
            continue
        name, sbits, vals, codes = [p.strip() for p in line[5:].split("|")]
        v = np.zeros(64, np.float32)
        for tok in vals.split():
            i, x = tok.split(":")
            v[int(i)] = np.float32(float(x))
        q = np.zeros(64, np.int8)
        for tok in codes.split():
            i, c = tok.split(":")
            q[int(i)] = int(c)
        cases.append((name, int(sbits, 16), v, q))
    return cases


@pytest.mark.parametrize("case", _parse_qsym_cases(), ids=lambda c: c[0])
def test_qsym64_golden(case):
    name, sbits, v, q = case
    s, codes = svdq.qsym64(v[None, :])
    assert numfmt.f16_bits(s)[0] == sbits
    assert np.array_equal(codes[0], q)


def test_pack_golden():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "int4_pack.txt")) if not l.startswith("#")]
    codes = np.array([int(t) for t in lines[0][1:]], np.int8)[None, :]
    exp = np.array([int(t, 16) for t in lines[1][1:]], np.uint8)[None, :]
    assert np.array_equal(svdq.pack_int4(codes), exp)
    assert np.array_equal(svdq.unpack_int4(exp), codes)


def test_pack_roundtrip_and_range():
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, size=(9, 128)).astype(np.int8)
    assert np.array_equal(svdq.unpack_int4(svdq.pack_int4(c)), c)
    with pytest.raises(ValueError):
        svdq.pack_int4(np.full((1, 2), -8, np.int8))


def _e2m3_value(f: int) -> float:
    """OCP E2M3 decode of one 6-bit field (bias 1; exponent 0 is subnormal)."""
    sign, exp, man = (f >> 5) & 1, (f >> 3) & 3, f & 7
    v = man / 8.0 if exp == 0 else (1.0 + man / 8.0) * 2.0 ** (exp - 1)
    return -v if sign else v


def test_pack_word_is_folded_e2m3_stream():
    """Unfold each stored word into the 96-bit stream of 16 E2M3 fields and
    decode every field as an FP6 value: it must be the code / 8 with a zero
    exponent, which is what the 4-bit MFMA operand expects."""
    exp_bits = [6 * e + 3 for e in range(16)] + [6 * e + 4 for e in range(16)]
    lo_mask = sum(1 << t for t in exp_bits if t < 32)
    hi_mask = sum(1 << (t - 64) for t in exp_bits if t >= 64)
    assert lo_mask & hi_mask == 0
    rng = np.random.default_rng(5)
    c = rng.integers(-7, 8, size=(3, 64)).astype(np.int8)
    words = svdq.pack_int4(c).view("<u8")
    for r in range(3):
        for w in range(4):
            x = int(words[r, w])
            x0, x1 = x & 0xFFFFFFFF, x >> 32
            t = (x0 & ~lo_mask & 0xFFFFFFFF) | (((x0 & lo_mask) | (x1 & hi_mask)) << 32) \
                | ((x1 & ~hi_mask & 0xFFFFFFFF) << 64)
            for e in range(16):
                f = (t >> (6 * e)) & 63
                assert (f >> 3) & 3 == 0
                assert _e2m3_value(f) * 8 == c[r, 16 * w + e]


def test_scale_layout_quad_major():
    """Format v3 scale storage, checked element by element on a hand-written
    case: G = 6 groups (one full quad and one half-filled quad) of 2 rows."""
    s = np.array([[1, 2, 3, 4, 5, 6], [7, 8, 9, 10, 11, 12]], np.float16)
    p = svdq.pack_scales(s)
    exp = np.array([[[1, 2, 3, 4], [7, 8, 9, 10]],
                    [[5, 6, 0, 0], [11, 12, 0, 0]]], np.float16)
    assert p.shape == (2, 2, 4) and np.array_equal(p, exp)
    # byte view: quad 1 of row 0 starts 2 rows * 8 bytes into the array
    assert p.tobytes()[16:18] == np.float16(5).tobytes()
    assert np.array_equal(svdq.unpack_scales(p, 6), s)
    rng = np.random.default_rng(3)
    for G in (1, 4, 7, 48):
        r = rng.standard_normal((5, G)).astype(np.float16)
        assert np.array_equal(svdq.unpack_scales(svdq.pack_scales(r), G), r)


def test_qsym64_error_bound_and_idempotence():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((4000, 64)) * np.exp(rng.uniform(-8, 8, (4000, 1)))).astype(np.float32)
    s, q = svdq.qsym64(v)
    sf = s.astype(np.float64)
    assert q.min() >= -7 and q.max() <= 7
    normal = sf >= 2.0 ** -14
    err = np.abs(v.astype(np.float64) - sf[:, None] * q)
    assert np.all(err[normal] <= (sf[normal] / 2 * (1 + 2.0 ** -10))[:, None])
    # the largest magnitude always maps to |q| = 7
    assert np.all(np.max(np.abs(q), axis=1)[normal] == 7)
    # re-quantising the dequantised group returns identical scale and codes
    deq = (sf[:, None] * q).astype(np.float32)
    s2, q2 = svdq.qsym64(deq)
    assert np.array_equal(numfmt.f16_bits(s2), numfmt.f16_bits(s)) and np.array_equal(q2, q)


def test_smoothing_closed_form():
    ax = np.array([4.0, 9.0, 0.0, 1.0], np.float32)
    aw = np.array([1.0, 4.0, 2.0, 0.0], np.float32)
    lam, inv = svdq.smoothing(ax, aw, 0.5)
    assert np.allclose(lam, [2.0, 1.5, 1.0, 1.0], rtol=0, atol=1e-15)
    assert np.array_equal(inv, np.float32([0.5, 1 / 1.5, 1.0, 1.0]))
    lam0, _ = svdq.smoothing(ax[:2], aw[:2], 1.0)      # alpha = 1: lambda = ax
    assert np.allclose(lam0, [4.0, 9.0])


def test_calib_absmax_hand_case():
    """Per input channel k: ax over the tokens of X [M, K], aw over the
    outputs of W [K, N]. Non-square shapes, and the largest-magnitude entry of
    most channels is negative, so a dropped abs() or a reduction over the
    wrong axis gives different numbers (or a different length)."""
    x = np.array([[1.0, -5.0, 2.0, 0.0],
                  [-3.0, 4.0, -7.0, 0.5],
                  [2.0, 1.0, 6.0, -0.25]], np.float32)          # M = 3, K = 4
    w = np.array([[-0.5, 0.25],
                  [0.125, -0.375],
                  [-0.25, 0.25],
                  [0.0, -0.0]], np.float32)                      # K = 4, N = 2
    ax, aw = svdq.calib_absmax(x, w)
    assert ax.shape == (4,) and aw.shape == (4,)
    assert ax.tolist() == [3.0, 5.0, 7.0, 0.5]
    assert aw.tolist() == [0.5, 0.375, 0.25, 0.0]
    assert ax.dtype == np.float32 and aw.dtype == np.float32


def test_prepare_uses_channel_maxima():
    """prepare_svdq's smoothing vector on a non-square layer (M 5, K 64,
    N 16) whose channel maxima are planted with negative signs: inv_lambda[k]
    = 1 / sqrt(ax[k] / aw[k]) by hand, and 1 where the weight row is zero."""
    rng = np.random.default_rng(7)
    M, K, N = 5, 64, 16
    x = numfmt.bf16_bits_to_f32(numfmt.f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (M, K)).astype(np.float32)))
    w = numfmt.bf16_bits_to_f32(numfmt.f32_to_bf16_bits(rng.uniform(-0.005, 0.005, (K, N)).astype(np.float32)))
    ax = np.ldexp(1.0, rng.integers(0, 4, K)).astype(np.float64)      # powers of two
    aw = np.ldexp(1.0, -rng.integers(5, 8, K)).astype(np.float64)
    for k in range(K):
        x[(3 * k) % M, k] = -ax[k]
        w[k, (5 * k) % N] = -aw[k]
    w[9, :] = 0.0
    xb = numfmt.f32_to_bf16_bits(x)
    wb = numfmt.f32_to_bf16_bits(w)
    assert np.array_equal(numfmt.bf16_bits_to_f32(xb), x) and np.array_equal(numfmt.bf16_bits_to_f32(wb), w)
    p = svdq.prepare_svdq(xb, wb, None, 0)
    lam = np.sqrt(ax / aw)
    lam[9] = 1.0
    assert np.array_equal(p.inv_lambda, (1.0 / lam).astype(np.float32))


def test_smoothing_preserves_product():
    """X_hat W_hat = X W (the migration changes nothing before quantisation)."""
    li = synth.make_layer(synth.CONFIGS["tiny"], M=64)
    x = numfmt.bf16_bits_to_f32(li.x)
    w = numfmt.bf16_bits_to_f32(li.w)
    ax, aw = svdq.calib_absmax(x, w)
    _, inv = svdq.smoothing(ax, aw, 0.5)
    x_hat = x.astype(np.float64) * inv.astype(np.float64)
    w_hat = svdq.smooth_weight(w, inv)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(x_hat @ w_hat - ref) <= 1e-12 * np.linalg.norm(ref)
    # outlier channels are the ones scaled down on the activation side
    assert np.all(inv[li.outlier_cols] < np.median(inv))


def _brute_y(qx, sx, qw, sw, xl1, l2, bias):
    M, K = qx.shape
    N = qw.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for g in range(K // 64):
                p = 0
                for k in range(64 * g, 64 * g + 64):
                    p += int(qx[m, k]) * int(qw[n, k])
                acc += float(sx[m, g]) * float(sw[n, g]) * p
            for j in range(xl1.shape[1]):
                acc += float(xl1[m, j]) * float(l2[j, n])
            y[m, n] = acc + float(bias[n])
    return y


def test_output_brute_force_tiny():
    rng = np.random.default_rng(2)
    M, K, N, r = 3, 192, 5, 4
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    sx = rng.uniform(0.01, 1, (M, K // 64)).astype(np.float16)
    sw = rng.uniform(0.01, 1, (N, K // 64)).astype(np.float16)
    xl1 = rng.standard_normal((M, r)).astype(np.float32)
    l2 = numfmt.f32_to_bf16_bits(rng.standard_normal((r, N)).astype(np.float32))
    b = numfmt.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    y = svdq.linear_output(qx, sx, qw, sw, xl1, l2, b)
    ref = _brute_y(qx, sx.astype(np.float64), qw, sw.astype(np.float64), xl1,
                   numfmt.bf16_bits_to_f32(l2), numfmt.bf16_bits_to_f32(b))
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    P = svdq.group_partials(qx, qw)
    for m in range(M):
        for n in range(N):
            for g in range(K // 64):
                assert P[m, n, g] == sum(int(qx[m, k]) * int(qw[n, k]) for k in range(64 * g, 64 * g + 64))


def test_grid_exact_layer():
    """Activations and residual placed exactly on the quantisation grid (power
    of two scales, every group reaching |q| = 7): the quantised layer equals
    the plain product of the original values plus bias."""
    rng = np.random.default_rng(3)
    M, K, N = 8, 256, 24
    qx = rng.integers(-7, 8, (M, K))
    qx[:, ::64] = 7
    ex = rng.integers(-6, 2, (M, K // 64))
    x_hat = (qx * np.repeat(2.0 ** ex, 64, axis=1)).astype(np.float32)
    qr = rng.integers(-7, 8, (N, K))
    qr[:, 1::64] = -7
    er = rng.integers(-10, -4, (N, K // 64))
    r_t = (qr * np.repeat(2.0 ** er, 64, axis=1)).astype(np.float32)    # [N, K]
    bias = numfmt.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    x_bits = numfmt.f32_to_bf16_bits(x_hat)
    assert np.array_equal(numfmt.bf16_bits_to_f32(x_bits), x_hat)       # exact in bf16
    qa = svdq.quantize_act(x_bits, None, None)
    codes_w, sw = svdq.quantize_rows(r_t)
    y = svdq.linear_output(qa.codes, qa.sx, codes_w, sw, qa.xl1, None, bias)
    ref = x_hat.astype(np.float64) @ r_t.astype(np.float64).T + numfmt.bf16_bits_to_f32(bias)
    assert np.array_equal(qa.codes, qx.astype(np.int8))
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_planted_low_rank_is_absorbed():
    """A weight of exact rank r (no smoothing): the low-rank branch takes all
    of it and the 4-bit residual only carries the bf16 rounding of L1, L2."""
    rng = np.random.default_rng(4)
    K, N, r, M = 256, 192, 8, 32
    w = (rng.standard_normal((K, r)) @ rng.standard_normal((r, N)) * 0.01).astype(np.float32)
    w_bits = numfmt.f32_to_bf16_bits(w)
    x_bits = synth.make_matrix_bf16(M, K, seed=9)
    wts = svdq.prepare_svdq(x_bits, w_bits, None, r, smooth=False)
    wf = numfmt.bf16_bits_to_f32(w_bits).astype(np.float64)
    assert np.linalg.norm(wts.sw.astype(np.float64)) * 7 <= 0.05 * np.linalg.norm(wf)
    _, y = svdq.forward(wts, x_bits)
    ref = numfmt.bf16_bits_to_f32(x_bits).astype(np.float64) @ wf
    assert np.linalg.norm(y - ref) <= 1e-2 * np.linalg.norm(ref)


def test_rank_zero_is_plain_w4a4():
    """Rank 0 without smoothing: codes and output equal plain W4A4 on (X, W)
    (activation and weight each quantised on their own, no extra terms)."""
    li = synth.make_layer(synth.CONFIGS["tiny"], M=32)
    wts = svdq.prepare_svdq(li.x, li.w, li.bias, 0, smooth=False)
    x = numfmt.bf16_bits_to_f32(li.x)
    w = numfmt.bf16_bits_to_f32(li.w)
    cw, sw = svdq.quantize_rows(np.ascontiguousarray(w.T))
    assert np.array_equal(wts.qw_codes, cw) and np.array_equal(wts.sw, sw)
    qa, y = svdq.forward(wts, li.x)
    cx, sx = svdq.quantize_rows(x)
    assert np.array_equal(qa.codes, cx) and qa.xl1.shape == (32, 0)
    deq = svdq.dequantize_rows(cx, sx) @ svdq.dequantize_rows(cw, sw).T
    ref = deq + numfmt.bf16_bits_to_f32(li.bias)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    # with smoothing, rank 0 is plain W4A4 on (X_hat, W_hat)
    wts_s = svdq.prepare_svdq(li.x, li.w, None, 0, smooth=True, keep_w_hat=True)
    cws, _ = svdq.quantize_rows(np.ascontiguousarray(wts_s.w_hat.T.astype(np.float32)))
    assert np.array_equal(wts_s.qw_codes, cws)


@pytest.fixture(scope="module")
def tiny_layer():
    cfg = synth.CONFIGS["tiny"]
    li = synth.make_layer(cfg)
    return cfg, li, svdq.prepare_svdq(li.x, li.w, li.bias, cfg.rank)


def test_svdq_beats_plain_w4a4_on_outliers(tiny_layer):
    """Method sanity (an expectation, not parity): with outlier channels, the
    smoothed + low-rank layer is closer to the exact layer than plain W4A4."""
    cfg, li, wts = tiny_layer
    _, y = svdq.forward(wts, li.x)
    plain = svdq.prepare_svdq(li.x, li.w, li.bias, 0, smooth=False)
    _, yp = svdq.forward(plain, li.x)
    ye = svdq.exact_output(li.x, li.w, li.bias)
    e_svdq = np.linalg.norm(y - ye) / np.linalg.norm(ye)
    e_plain = np.linalg.norm(yp - ye) / np.linalg.norm(ye)
    assert e_svdq < 0.5 * e_plain


def test_lowrank_branch_carries_leading_energy(tiny_layer):
    cfg, li, wts = tiny_layer
    w = numfmt.bf16_bits_to_f32(li.w)
    ax, aw = svdq.calib_absmax(numfmt.bf16_bits_to_f32(li.x), w)
    _, inv = svdq.smoothing(ax, aw, 0.5)
    w_hat = svdq.smooth_weight(w, inv)
    ref = np.linalg.svd(w_hat, compute_uv=False)
    res = np.linalg.norm(w_hat - numfmt.bf16_bits_to_f32(wts.l1).astype(np.float64)
                         @ numfmt.bf16_bits_to_f32(wts.l2).astype(np.float64)) ** 2
    assert res <= 1.03 * np.sum(ref[cfg.rank:] ** 2)


def test_gelu_tanh_values():
    assert svdq.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(svdq.gelu_tanh(np.array([1.0]))[0] - 0.8411919906082768) < 1e-15
    x = np.linspace(-6, 6, 241)
    g = svdq.gelu_tanh(x)
    assert np.allclose(g - svdq.gelu_tanh(-x), x, atol=1e-14)          # g(x) - g(-x) = x
    erf_gelu = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in x])
    assert np.max(np.abs(g - erf_gelu)) < 1e-3                          # tanh form approximates erf form
    assert abs(svdq.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12


def test_l1_tile_layout_hand_case_and_roundtrip():
    """The L1 tile layout (format v4): element (g, t, s, l, j) of the flat
    array is L1[64 g + 16 (l // 16) + 8 s + j, 16 t + l % 16]. Values that
    encode their own (k, rank) position make every slot checkable by hand."""
    K, r = 128, 32
    l1 = (np.arange(K)[:, None] * 256 + np.arange(r)[None, :]).astype(np.uint16)   # = 256 k + n
    p = svdq.pack_l1_tiles(l1)
    assert p.shape == (K * r,)
    # first 1 KB: g 0, t 0, s 0; lane 0 holds k 0..7 of rank 0, lane 17 k 16..23 of rank 1
    assert p[0:8].tolist() == [256 * k for k in range(8)]
    assert p[17 * 8:18 * 8].tolist() == [256 * k + 1 for k in range(16, 24)]
    # step 1 of the same tile: lane 63 holds k 56..63 of rank 15
    base = 512
    assert p[base + 63 * 8:base + 64 * 8].tolist() == [256 * k + 15 for k in range(56, 64)]
    # tile t = 1 of group 0 (ranks 16..31), then group 1 (k 64..127)
    assert p[2 * 512:2 * 512 + 8].tolist() == [256 * k + 16 for k in range(8)]
    assert p[4 * 512 + 5 * 8:4 * 512 + 6 * 8].tolist() == [256 * k + 5 for k in range(64, 72)]
    rng = np.random.default_rng(2)
    for K2, r2 in [(64, 16), (320, 48), (3072, 128)]:
        a = rng.integers(0, 65536, (K2, r2)).astype(np.uint16)
        assert np.array_equal(svdq.unpack_l1_tiles(svdq.pack_l1_tiles(a), K2, r2), a)


def test_library_l1_packer_matches_oracle():
    """The package's pack_l1 (torch indexing) and the oracle's packer (loops
    over the definition) are written apart; they must agree."""
    import torch
    import bit_quantized_diffusion_svdq_amd as lib
    rng = np.random.default_rng(3)
    for K, r in [(64, 16), (320, 48), (3072, 32), (1024, 128)]:
        a = rng.integers(0, 65536, (K, r)).astype(np.uint16)
        got = lib.pack_l1(torch.from_numpy(a.view(np.int16))).numpy().view(np.uint16)
        assert np.array_equal(got, svdq.pack_l1_tiles(a)), (K, r)
    with pytest.raises(ValueError):
        lib.pack_l1(torch.zeros((96, 16), dtype=torch.int16))
