"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against the OCP MX definitions
and hand-derived cases; CPU only."""
import numpy as np
import pytest

from oracle import mxfp4 as mx


def _e2m1_decode(nib: int) -> float:
    """E2M1 from its bits (sign bit 3, exponent bits 1-2, mantissa bit 0,
    exponent bias 1, exponent 0 = subnormal), independent of the grid table."""
    s, e, m = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    v = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


def test_grid_is_e2m1_encoding():
    for k in range(8):
        assert _e2m1_decode(k) == mx.E2M1_GRID[k]
        assert _e2m1_decode(8 | k) == -mx.E2M1_GRID[k]


@pytest.mark.parametrize("t,code", [
    (0.0, 0), (0.2, 0), (0.25, 0), (0.26, 1), (0.5, 1), (0.75, 2), (1.2, 2), (1.25, 2),
    (1.3, 3), (1.75, 4), (2.5, 4), (2.6, 5), (3.5, 6), (4.9, 6), (5.0, 6), (5.1, 7),
    (6.0, 7), (7.9, 7), (100.0, 7), (-0.1, 0), (-0.3, -1), (-2.5, -4), (-5.0, -6), (-9.0, -7),
])
def test_e2m1_round_hand_cases(t, code):
    """Nearest E2M1 value; ties (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) go to
    the even index (mantissa bit 0); beyond 6 saturates; -0 is stored as 0."""
    assert int(mx.e2m1_round(np.array([t]))[0]) == code


@pytest.mark.parametrize("amax,e", [
    (6.0, 0), (7.0, 0), (7.99, 0), (8.0, 1), (4.0, 0), (3.99, -1), (0.3, -4), (1.0, -2),
    (0.0, -127), (2.0 ** -140, -127), (2.0 ** 200, 127), (1.5 * 2.0 ** 10, 8),
])
def test_block_exponent_hand_cases(amax, e):
    """e = floor(log2(amax)) - 2, clamped to the E8M0 range; 0 -> -127."""
    assert int(mx.block_exponent(np.array([amax]))[0]) == e


def test_quantize_block_hand_case():
    v = np.zeros((1, 32), np.float32)
    v[0, :4] = [7.0, -0.3, 2.5, 3.0]           # amax 7 -> e = 0, values used as is
    codes, e = mx.quantize_rows(v)
    assert e.tolist() == [[0]]
    assert codes[0, :4].tolist() == [7, -1, 4, 5] and not codes[0, 4:].any()
    v2 = v * 2.0 ** -5                          # same block scaled: e = -5, same codes
    codes2, e2 = mx.quantize_rows(v2)
    assert e2.tolist() == [[-5]] and np.array_equal(codes2, codes)


def test_error_bound_and_idempotence():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    codes, e = mx.quantize_rows(v)
    d = mx.dequantize_rows(codes, e)
    X = np.repeat(np.ldexp(1.0, e.astype(np.int64)), 32, axis=1)
    err = np.abs(v.astype(np.float64) - d)
    assert np.all(err <= 2 * X)                               # saturation 8 -> 6 is the worst case
    inside = np.abs(v) <= 6 * X
    assert np.all(err[inside] <= X[inside])                   # half the widest spacing (2)
    # requantising the dequantised values gives the same codes (e may only drop)
    c2, e2 = mx.quantize_rows(d.astype(np.float32))
    assert np.array_equal(mx.dequantize_rows(c2, e2), d)


def test_pack_fp4_hand_bytes_and_roundtrip():
    c = np.array([[1, -1, 7, -7, 0, 4]], np.int8)
    assert mx.pack_fp4(c).tolist() == [[0x91, 0xF7, 0x40]]
    rng = np.random.default_rng(1)
    r = rng.integers(-7, 8, (5, 64)).astype(np.int8)
    assert np.array_equal(mx.unpack_fp4(mx.pack_fp4(r)), r)


def test_scale_layout_hand_case():
    """10 blocks of one row: quad 0 holds blocks 0..7 as [0 2 4 6 | 1 3 5 7],
    quad 1 blocks 8, 9 at bytes 0 and 4, the rest 0."""
    e = np.arange(10, dtype=np.int16)[None, :] - 3         # exponents -3 .. 6
    p = mx.pack_scales(e)
    assert p.shape == (2, 1, 8)
    assert p[0, 0].tolist() == [124, 126, 128, 130, 125, 127, 129, 131]
    assert p[1, 0].tolist() == [132, 0, 0, 0, 133, 0, 0, 0]
    assert np.array_equal(mx.unpack_scales(p, 10), e)


def test_linear_output_brute_force_tiny():
    rng = np.random.default_rng(7)
    M, K, N, r = 3, 64, 5, 2
    a = rng.integers(-7, 8, (M, K)).astype(np.int8)
    w = rng.integers(-7, 8, (N, K)).astype(np.int8)
    ea = rng.integers(-6, 3, (M, K // 32)).astype(np.int16)
    ew = rng.integers(-6, 3, (N, K // 32)).astype(np.int16)
    xl1 = rng.standard_normal((M, r)).astype(np.float32)
    l2 = (rng.standard_normal((r, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bias = (rng.standard_normal(N).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = mx.linear_output(a, ea, w, ew, xl1, l2, bias)

    def val(c, e):
        return (-1 if c < 0 else 1) * _e2m1_decode(abs(int(c))) * 2.0 ** int(e)

    def bf(b):
        return float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += val(a[m, k], ea[m, k // 32]) * val(w[n, k], ew[n, k // 32])
            for j in range(r):
                s += float(xl1[m, j]) * bf(l2[j, n])
            s += bf(bias[n])
            assert abs(y[m, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_mx_layer_close_to_exact_and_rank_helps():
    """Method sanity: the MXFP4 SVDQ layer tracks X W, and the low-rank branch
    lowers the error on outlier inputs."""
    import synth
    from oracle import svdq
    cfg = synth.CONFIGS["tiny"]
    li = synth.make_layer(cfg)
    ex = svdq.exact_output(li.x, li.w, li.bias)
    errs = []
    for rank in (0, cfg.rank):
        w = mx.prepare_mx(li.x, li.w, li.bias, rank)
        _, y = mx.forward(w, li.x)
        errs.append(np.linalg.norm(y - ex) / np.linalg.norm(ex))
    assert errs[1] < errs[0] < 0.2
