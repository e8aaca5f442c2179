// Device helpers that turn fp32 values into stored INT4 codes (format v2):
// one code as its FP6 E2M3 field, and sixteen fields folded into the 64-bit
// storage word. Shared by the activation kernel and the offline residual
// quantiser, which store codes the same way.
#pragma once
#include "common.h"

// Quantise one value given the group's fp32 reciprocal `inv` (0 when the
// scale is 0) and return its FP6 E2M3 field: magnitude in bits 0-2, zero
// exponent, sign in bit 5 (zero is stored with sign 0). Clamping to [-7, 7]
// before rounding equals clamping after it (the bounds are integers);
// |a| + 1.5 * 2^23 rounds |a| half-to-even into the low mantissa bits (the
// spacing there is 1 and the constant is even), and round(a) < 0 exactly
// when a + 0.5 < 0, which gives the sign without a compare.
DEV uint32_t code_field(float v, float inv) {
    const float t = v * inv;                   // one fp32 multiply (no contraction)
    const float a = __builtin_amdgcn_fmed3f(t, -7.0f, 7.0f);
    const uint32_t mag = __float_as_uint(fabsf(a) + 12582912.0f) & 7u;
    const uint32_t sgn = (__float_as_uint(a + 0.5f) >> 26) & 32u;
    return mag | sgn;
}

// Sixteen E2M3 fields (code e at bits 6e..6e+5 of a 96-bit stream T) -> the
// 64-bit storage word: T[0:32) and T[64:96) keep their places, and the bits of
// T[32:64) go into the zero exponent positions of those two thirds
// (0x18618618 in the low word, 0x61861861 in the high word).
DEV uint2 fold_fields(const uint32_t (&f)[16]) {
    const uint32_t d0 = f[0] | (f[1] << 6) | (f[2] << 12) | (f[3] << 18) | (f[4] << 24) | (f[5] << 30);
    const uint32_t d1 = (f[5] >> 2) | (f[6] << 4) | (f[7] << 10) | (f[8] << 16) | (f[9] << 22) | (f[10] << 28);
    const uint32_t d2 = (f[10] >> 4) | (f[11] << 2) | (f[12] << 8) | (f[13] << 14) | (f[14] << 20) | (f[15] << 26);
    return make_uint2(d0 | (d1 & 0x18618618u), d2 | (d1 & 0x61861861u));
}
