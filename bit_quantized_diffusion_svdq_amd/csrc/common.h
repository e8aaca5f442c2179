// Shared device helpers for the gfx950 kernels (vector types, MFMA wrappers,
// bf16/fp16 bit conversions). Written for CDNA4 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

#define DEV __device__ __forceinline__

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3: 32-bit data
// format, no swizzle). Loads beyond `bytes` return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
DEV rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

DEV float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
DEV float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (gfx950 has a native convert).
DEV uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

DEV uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

DEV float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// D = A(32x64 fp8) * B(64x32 fp8) + C, fp32 accumulate. Both operands carry
// INT4 codes as E4M3 subnormals (value q * 2^-9, see int4sm_to_fp8); the
// E8M0 block scale 2^9 (0x88) on each side turns the products back into
// exact integer products, so the result is the exact integer dot product.
DEV v16f mfma_f8_32x32x64(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x88888888, 0, 0x88888888);
}

// D = A(16x32 bf16) * B(32x16 bf16) + C
DEV v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16 bf16) * B(16x32 bf16) + C
DEV v16f mfma_bf16_32x32x16(const v8bf& a, const v8bf& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16 f16) * B(16x32 f16) + C
DEV v16f mfma_f16_32x32x16(const v8h& a, const v8h& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Eight sign-magnitude INT4 codes (one dword, element 2i in the low nibble of
// byte i) -> eight FP8 E4M3 bytes. A code s|m (sign bit, magnitude 0..7)
// becomes the E4M3 subnormal s|0000|m, whose value is (-1)^s * m * 2^-9, so
// the byte is just the magnitude bits with the sign moved to bit 7.
// lo: bytes = elements 0,2,4,6; hi: bytes = elements 1,3,5,7. Operands A and
// B are expanded the same way, so the K order inside an MFMA is permuted
// identically on both sides and every dot product is unchanged.
DEV void int4sm_to_fp8(uint32_t x, uint32_t& lo, uint32_t& hi) {
    lo = (x & 0x07070707u) | ((x << 4) & 0x80808080u);
    hi = ((x >> 4) & 0x07070707u) | (x & 0x80808080u);
}

DEV float gelu_tanh_f32(float y) {
    const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
    const float k1 = 0.044715f;
    float u = k0 * (y + k1 * y * y * y);
    return 0.5f * y * (1.0f + tanhf(u));
}
