"""Pins for the oracle's rounding helpers (bf16 RTNE, fp16)."""
import numpy as np
import pytest
import torch

from oracle import numfmt


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_all_upper_halves_with_rounding_tails():
    """Every upper 16-bit pattern combined with every rounding-relevant tail
    (zero, 1, below/at/above the halfway point, all ones) against torch's
    float32 -> bfloat16 conversion (an independent RTNE implementation)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    tails = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = (hi[:, None] | tails[None, :]).ravel()
    f = bits.view(np.float32)
    mine = numfmt.f32_to_bf16_bits(f)
    ref = _torch_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(mine[~nan], ref[~nan])
    # NaN stays NaN (quiet bit set), sign kept
    back = numfmt.bf16_bits_to_f32(mine[nan])
    assert np.isnan(back).all()


def test_bf16_random_patterns():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    ok = ~np.isnan(f)
    assert np.array_equal(numfmt.f32_to_bf16_bits(f)[ok], _torch_bf16_bits(f)[ok])


def test_bf16_known_values():
    f = np.array([1.0, -2.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.3895313892515355e38,
                  3.4e38, 2 ** -133, 2 ** -134], np.float32)
    exp = np.array([0x3F80, 0xC000, 0x3F80, 0x3F82, 0x7F7F, 0x7F80, 0x0001, 0x0000], np.uint16)
    assert np.array_equal(numfmt.f32_to_bf16_bits(f), exp)


def test_f64_to_bf16_single_rounding():
    # 1 + 2^-8 + 2^-30: above the bf16 halfway point, so it rounds up to
    # 1 + 2^-7 (0x3F81). Rounding through float32 first would land exactly on
    # the halfway point 1 + 2^-8 and then round to even, 1.0 (0x3F80).
    y = np.array([1.0 + 2 ** -8 + 2 ** -30, 1.0 + 2 ** -8, -(1.0 + 2 ** -8 + 2 ** -30)])
    assert list(numfmt.f64_to_bf16_bits(y)) == [0x3F81, 0x3F80, 0xBF81]
    assert numfmt.f32_to_bf16_bits(np.float32(y[0])) == 0x3F80


def test_f64_to_bf16_agrees_with_f32_path_when_exact():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(numfmt.f64_to_bf16_bits(f.astype(np.float64)),
                          numfmt.f32_to_bf16_bits(f))
    assert numfmt.f64_to_bf16_bits(np.array([1e39, -1e39]))[0] == 0x7F80
    assert numfmt.f64_to_bf16_bits(np.array([np.nan]))[0] == 0x7FC0


@pytest.mark.parametrize("val,bits", [(65504.0, 0x7BFF), (65520.0, 0x7C00), (2.0 ** -24, 0x0001),
                                      (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002),
                                      (1.0 / 3.0, 0x3555), (0.1, 0x2E66)])
def test_f16_known_values(val, bits):
    assert numfmt.f16_bits(numfmt.f32_to_f16(np.float32(val))) == bits
