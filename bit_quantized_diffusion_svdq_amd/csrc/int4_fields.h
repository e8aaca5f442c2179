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

// The same 64-bit storage word from sixteen values on the hardware FP6
// conversion. t = v * (inv / 8) is the value in code units over 8 (scaling by
// 2^-3 is exact here, and a product too small for that rounds to code 0 on
// both routes), clamped to +-7/8; v_cvt_scalef32_2xpk16_fp6_f32 with scale 1
// rounds it to the E2M3 grid, whose subnormals are exactly the multiples of
// 1/8 up to 7/8, half to even: the result is the code's E2M3 field. The
// instruction takes field 2j from its first source's element j and field
// 2j + 1 from its second's, and keeps the sign of a value that rounds to
// zero; those signs are cleared (a field's magnitude + 7 carries into its
// zero exponent bit exactly when the magnitude is nonzero), then the stream
// is folded as by fold_fields. Bit-identical to code_field + fold_fields.
DEV uint2 codes16_fp6(const float* v, float inv) {
    typedef float v8f __attribute__((ext_vector_type(8)));
    typedef uint32_t v6u __attribute__((ext_vector_type(6)));
    const float inv8 = inv * 0.125f;
    v8f ev, od;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ev[j] = __builtin_amdgcn_fmed3f(v[2 * j] * inv8, -0.875f, 0.875f);
        od[j] = __builtin_amdgcn_fmed3f(v[2 * j + 1] * inv8, -0.875f, 0.875f);
    }
    const v16f a = __builtin_shufflevector(ev, ev, 0, 1, 2, 3, 4, 5, 6, 7, -1, -1, -1, -1, -1, -1, -1, -1);
    const v16f b = __builtin_shufflevector(od, od, 0, 1, 2, 3, 4, 5, 6, 7, -1, -1, -1, -1, -1, -1, -1, -1);
    const v6u r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
    // fields 0-9 and the low four bits of field 10 in lo; the rest of field
    // 10 (exponent bit, sign at bit 1) and fields 11-15 (from bit 2) in hi
    uint64_t lo = (uint64_t)r[0] | ((uint64_t)r[1] << 32);
    uint32_t hi = r[2];
    const uint64_t nz = ((lo & 0x71c71c71c71c71c7ull) + 0x71c71c71c71c71c7ull) & 0x8208208208208208ull;
    lo &= ~0x0820820820820820ull | (nz << 2);
    const uint32_t nzh = ((hi & 0x1c71c71cu) + 0x1c71c71cu) & 0x20820820u;
    hi &= ~0x82082082u | (nzh << 2) | ((uint32_t)(nz >> 62) & 2u);
    const uint32_t d0 = (uint32_t)lo, d1 = (uint32_t)(lo >> 32);
    return make_uint2(d0 | (d1 & 0x18618618u), hi | (d1 & 0x61861861u));
}
