// Shared device helpers for the gfx950 kernels (vector types, MFMA wrappers,
// bf16/fp16 bit conversions). Written for CDNA4 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
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

// D = A(32x64) * B(64x32) + C with both operands FP6 E2M3 (cbsz = blgp = 2):
// 32 six-bit fields per lane packed at 6-bit strides in 6 dwords. A 4-bit code q is the E2M3 subnormal q / 8
// (zero exponent) and the E8M0 block scale 2^3 (0x82) on each side restores
// q_a * q_w, so the fp32 result is the exact integer dot product (|sum| <= 3136).
DEV v16f mfma_fp6_32x32x64(const v6i& a, const v6i& b, const v16f& c) {
    const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, -1, -1);
    const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 2, 2, 0, 0x82828282, 0, 0x82828282);
}

// D = A(32x64) * B(64x32) + C with both operands MXFP4: 32 E2M1 codes per lane
// (4 dwords, code t at bits 4t), lane l holding row (or column) l % 32 and K
// block l / 32, each lane scaled by its own E8M0 byte, byte OA / OB of sa / sb
// (OCP MX block scales applied by the matrix pipe).
template <int OA, int OB>
DEV v16f mfma_mxfp4_32x32x64(const v4i& a, const v4i& b, const v16f& c, int sa, int sb) {
    const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
    const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OA, sa, OB, sb);
}

// Empty register ties: they emit no instruction, but code that uses the
// value afterwards cannot be scheduled above them, which keeps independent
// MFMAs in program order instead of being hoisted (and their results kept
// live) by the compiler.
template <class T>
DEV void order_point(T& x) { asm volatile("" : "+v"(x)); }
template <class T, class U>
DEV void order_point(T& x, U& y) { asm volatile("" : "+v"(x), "+v"(y)); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt) but, unlike __syncthreads(), not for its outstanding global
// loads, so prefetches stay in flight across it. The memory clobber keeps
// the compiler from moving memory accesses across the barrier.
DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// D = A(16x32 bf16) * B(32x16 bf16) + C
DEV v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16 bf16) * B(16x32 bf16) + C
DEV v16f mfma_bf16_32x32x16(const v8bf& a, const v8bf& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x8 f16) * B(8x32 f16) + C (same issue cost as the 32x32x16 form
// on gfx950, half the operand registers)
DEV v16f mfma_f16_32x32x8(const v4h& a, const v4h& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, c, 0, 0, 0);
}

// One stored 64-bit word of 16 codes (x0 = bits 0-31, x1 = bits 32-63) -> the
// three dwords of its E2M3 operand stream. The word keeps stream dwords 0 and
// 2 in place and carries stream dword 1 in their zero exponent fields, at
// 0x18618618 (low word) and 0x61861861 (high word).
DEV void unfold_fp6(uint32_t x0, uint32_t x1, uint32_t& d0, uint32_t& d1, uint32_t& d2) {
    d0 = x0 & ~0x18618618u;
    d1 = (x0 & 0x18618618u) | (x1 & 0x61861861u);
    d2 = x1 & ~0x61861861u;
}

// GELU, tanh form: 0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)), this is y / (1 + 2^t) with
// t = -2 u log2(e) = y (c1 + c2 y^2), c1 = -2 sqrt(2/pi) log2(e) and
// c2 = 0.044715 c1 (fp32 roundings of those products): one v_exp_f32 (2^t)
// and one v_rcp_f32. Large negative y: 2^t overflows to inf and the result is
// -0; large positive y: 2^t -> 0 and the result is y. The error is a few fp32
// ulps of the result, plus about an ulp of |y| far in the negative tail,
// where the function itself is below 1e-28 (the 1 + tanh form cancels there).
DEV float gelu_tanh_f32(float y) {
    const float c1 = -2.302208185195923f, c2 = -0.10294324159622192f;
    const float t = y * __builtin_fmaf(c2, y * y, c1);
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// Eight E2M1 nibbles (t[0] in bits 0-3): round to nearest, ties to mantissa
// 0, saturating at 6 (the conversion instruction), then the sign of every
// zero nibble cleared: (mag + 7) carries into bit 3 exactly when mag != 0.
DEV uint32_t e2m1_x8(const float* t) {
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[0], t[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[2], t[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[4], t[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[6], t[7], 1.0f, 3);
    const uint32_t nonzero = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;
    return w & (0x77777777u | nonzero);
}

// E8M0 block exponent of an MX block with absolute maximum amax (OCP
// Microscaling Formats v1.0: floor(log2 amax) minus the E2M1 emax of 2),
// read off the exponent field; a zero or subnormal amax clamps to -127.
DEV int mx_block_exponent(float amax) {
    const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xffu);
    return ebits - 129 < -127 ? -127 : ebits - 129;
}

// 2^-e for an E8M0 exponent e in [-127, 127], exact
DEV float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
