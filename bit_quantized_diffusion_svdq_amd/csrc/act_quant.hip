// svdq_quantize_act kernel: smoothing + rank-r down-projection + symmetric
// INT4 group-64 quantisation of the activations, in one pass over X.
//
// The fusion of the low-rank down-projection with input quantisation is the
// one the remio.ai page attributes to the original Nunchaku engine (section
// "SVDQuant moves hard values out of 4-bit"); here it is re-derived for CDNA4:
//  - one workgroup owns 16 token rows; its waves (16 for ranks up to 32,
//    else 8, as registers allow) take the 64-wide groups of K round-robin, so
//    every row is read from HBM exactly once with 128-byte contiguous row
//    segments per group; each wave issues the loads of two (with 16 waves)
//    or six of its groups at once (and the L1 fragments one group ahead)
//    before it quantises them, to keep enough bytes in flight for HBM while
//    a SIMD always has some wave whose data has landed;
//  - a lane holds 16 consecutive channels of one row (two dwordx4 loads);
//    the four lanes of a row (lanes l, l^16, l^32, l^48) reduce the group
//    absmax with two cross-lane max steps;
//  - the same registers feed the down-projection on the bf16 MFMA
//    (16x16x32), with X_hat split into bf16 hi + lo so the product keeps
//    ~16 mantissa bits; L1 arrives in a tile layout in which the B operand
//    of every (group, 16-rank tile, 32-channel step) is 1 KB in lane order
//    (lane l holds channels 16 (l / 16) + 8 step .. + 7 of rank l % 16, the
//    channels its A operand holds), so each L1 load is one contiguous 1 KB;
//  - per-wave fp32 partials of X_hat L1 are reduced across the waves in LDS
//    in a fixed order (deterministic, no atomics).
// The MXFP4 form (FMT 1) shares all of this and differs in the per-value
// step: a 32-value block spans two lanes (l, l ^ 16); its E8M0 exponent is
// floor(log2(amax)) - 2 clamped to [-127, 127], read off the exponent field
// of amax; each value is scaled by the exact power of two 2^-e and rounded to
// the nearest E2M1 value (ties to mantissa 0, saturating at 6) by
// v_cvt_scalef32_pk_fp4_f32 with scale 1 (OCP Microscaling Formats v1.0:
// E2M1, E8M0, conversion from FP32). The instruction keeps the sign of values
// that round to zero; those nibbles get sign 0 afterwards.
#include "common.h"

namespace {

constexpr int ROWS = 16;
// waves per workgroup: 16 (four per SIMD) while the rank leaves room in 128
// VGPRs (rank <= 32), else 8; more waves with fewer groups in flight each let a
// SIMD work on whichever wave's data has landed
__host__ __device__ constexpr int waves_for(int rt) { return rt <= 2 ? 16 : 8; }

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

// RT = rank / 16 (0..8); FMT 0: INT4 g64, 1: MXFP4; CHT: groups each wave
// keeps in flight (0: the default for the wave count)
template <int RT, int FMT, int CHT>
__global__ __launch_bounds__(waves_for(RT) * 64) void act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ inv_lambda, const uint16_t* __restrict__ l1t,
    uint8_t* __restrict__ qx, uint16_t* __restrict__ sx, float* __restrict__ xl1)
{
    constexpr int RTX = RT > 0 ? RT : 1;
    constexpr int WAVES = waves_for(RT), NTH = WAVES * 64;
    extern __shared__ float smem[];
    const int G = (int)(K / 64);
    float* s_inv = smem;                                   // [K]
    uint16_t* s_sx = (uint16_t*)(smem + K);                // [ROWS][G] fp16, or [ROWS][2G] E8M0 bytes
    float* s_xl1 = smem + K + ((ROWS * G + 1) / 2);        // [WAVES][ROWS][16*RT]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * ROWS;

    const int r = lane & 15, p = lane >> 4;
    const int64_t row = m0 + r;
    const bool valid = row < M;
    // rows past the end read the last row; nothing of theirs is stored
    const uint16_t* xrow = x + (valid ? row : M - 1) * ldx;
    // this wave's groups are wave, wave + WAVES, ...; indices past the end are
    // clamped to a real group so prefetches stay in bounds
    const int n = (G > wave) ? (G - wave + WAVES - 1) / WAVES : 0;
    auto gidx = [&](int i) { const int gi = wave + WAVES * i; return gi < G ? gi : G - 1; };

    v4f acc[RTX];
#pragma unroll
    for (int t = 0; t < RTX; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    auto loadx = [&](uint4 (&d)[2], int i) {
        const int kb = gidx(i) * 64 + 16 * p;
        d[0] = *(const uint4*)(xrow + kb);
        d[1] = *(const uint4*)(xrow + kb + 8);
    };
    // L1 in its tile layout: the B fragments of (group, rank tile, step) are
    // 1 KB in lane order, so each load instruction reads one contiguous
    // kilobyte (a [rank][K] layout touches 16 rows per instruction, which
    // costs the load pipe about twice as much)
    auto loadl = [&](v8bf (&d)[RTX][2], int i) {
        if constexpr (RT > 0) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const uint16_t* lf = l1t + ((int64_t)(gidx(i) * RT + t) * 2) * 512 + lane * 8;
                d[t][0] = *(const v8bf*)(lf);
                d[t][1] = *(const v8bf*)(lf + 512);
            }
        }
    };
    // quantise the lane's 16 values of group gidx(i) and feed the MFMA
    auto process = [&](const uint4 (&xv)[2], const v8bf (&lv)[RTX][2], int i) {
        const int g = gidx(i);
        const int kb = g * 64 + 16 * p;
        const uint32_t w[8] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w, xv[1].x, xv[1].y, xv[1].z, xv[1].w};
        float v[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[2 * j] = bf16_lo_to_f32(w[j]) * s_inv[kb + 2 * j];
            v[2 * j + 1] = bf16_hi_to_f32(w[j]) * s_inv[kb + 2 * j + 1];
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        if constexpr (FMT == 0) {
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const float s32 = fminf(amax / 7.0f, 65504.0f);
            const _Float16 s16 = (_Float16)s32;
            const float sf = (float)s16;
            const float inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;

            uint32_t f[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) f[j] = code_field(v[j], inv);
            const uint2 word = fold_fields(f);
            if (valid) {
                *(uint2*)(qx + row * (K / 2) + g * 32 + 8 * p) = word;
                if (p == 0) s_sx[r * G + g] = __builtin_bit_cast(uint16_t, s16);
            }
        } else {
            // block 2g + (p >> 1) of the row; e = floor(log2 amax) - 2 from the
            // exponent field (a zero or subnormal amax clamps to -127)
            const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xffu);
            const int e = ebits - 129 < -127 ? -127 : ebits - 129;
            const float sc = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
            float t[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) t[j] = v[j] * sc;
            const uint32_t lo = e2m1_x8(t), hi = e2m1_x8(t + 8);
            if (valid) {
                *(uint2*)(qx + row * (K / 2) + g * 32 + 8 * p) = make_uint2(lo, hi);
                if ((p & 1) == 0) ((uint8_t*)s_sx)[r * 2 * G + 2 * g + (p >> 1)] = (uint8_t)(e + 127);
            }
        }

        if constexpr (RT > 0) {
            // X_hat split into bf16 hi + lo; step 0 uses v[0..7], step 1 v[8..15].
            v8bf ah0, al0, ah1, al1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const __bf16 h0 = (__bf16)v[j];
                const __bf16 h1 = (__bf16)v[8 + j];
                ah0[j] = h0;
                ah1[j] = h1;
                al0[j] = (__bf16)(v[j] - (float)h0);
                al1[j] = (__bf16)(v[8 + j] - (float)h1);
            }
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                acc[t] = mfma_bf16_16x16x32(ah0, lv[t][0], acc[t]);
                acc[t] = mfma_bf16_16x16x32(al0, lv[t][0], acc[t]);
                acc[t] = mfma_bf16_16x16x32(ah1, lv[t][1], acc[t]);
                acc[t] = mfma_bf16_16x16x32(al1, lv[t][1], acc[t]);
            }
        }
    };

    // the X loads of up to CH groups are all issued before any is processed
    // (by default 16 waves x 2 groups or 8 x 6: 32 or 48 KB per CU in flight);
    // L1 fragments run one group ahead
    constexpr int CH = CHT ? CHT : (WAVES == 16 ? 2 : 6);
    static_assert(CH % 2 == 0, "groups are processed in pairs");
    v8bf la[RTX][2], lb[RTX][2];
    for (int c0 = 0; c0 < ((n + CH - 1) / CH) * CH || c0 == 0; c0 += CH) {
        uint4 xs[CH][2];
#pragma unroll
        for (int u = 0; u < CH; ++u) loadx(xs[u], c0 + u);
        loadl(la, c0);
        if (c0 == 0) {
            // the smoothing reciprocals go to LDS while the first X loads fly
            for (int64_t k = 4 * tid; k < K; k += 4 * NTH)
                *(float4*)(s_inv + k) = inv_lambda ? *(const float4*)(inv_lambda + k)
                                                   : make_float4(1.f, 1.f, 1.f, 1.f);
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < CH; u += 2) {
            if (c0 + u < n) {
                loadl(lb, c0 + u + 1);
                process(xs[u], la, c0 + u);
            }
            if (c0 + u + 1 < n) {
                loadl(la, c0 + u + 2);
                process(xs[u + 1], lb, c0 + u + 1);
            }
        }
    }

    if constexpr (RT > 0) {
        // C layout (16x16): lane holds column (lane & 15), rows 4 * (lane >> 4) + i.
        const int RK = 16 * RT;
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_xl1[(wave * ROWS + 4 * p + i) * RK + 16 * t + r] = acc[t][i];
    }
    __syncthreads();

    // scales, quad-major [G4][M][8 bytes]: quad q of the block's rows is one
    // contiguous 8 * ROWS-byte segment; groups past the last one are 0. INT4:
    // four fp16 scales per record; MXFP4: eight E8M0 bytes, even blocks first
    const int G4 = (G + 3) / 4;
    if constexpr (FMT == 0) {
        for (int e = tid; e < ROWS * G4 * 4; e += NTH) {
            const int q = e / (ROWS * 4), rr = (e / 4) % ROWS, gg = 4 * q + (e & 3);
            if (m0 + rr < M)
                sx[((int64_t)q * M + m0 + rr) * 4 + (e & 3)] = gg < G ? s_sx[rr * G + gg] : (uint16_t)0;
        }
    } else {
        const uint8_t* se = (const uint8_t*)s_sx;
        uint8_t* sxb = (uint8_t*)sx;
        const int nb = 2 * G;
        for (int e = tid; e < ROWS * G4 * 8; e += NTH) {
            const int q = e / (ROWS * 8), rr = (e / 8) % ROWS, idx = e & 7;
            const int b = 8 * q + 2 * (idx & 3) + (idx >> 2);
            if (m0 + rr < M)
                sxb[((int64_t)q * M + m0 + rr) * 8 + idx] = b < nb ? se[rr * nb + b] : (uint8_t)0;
        }
    }
    if constexpr (RT > 0) {
        const int RK = 16 * RT;
        for (int e = tid; e < ROWS * RK; e += NTH) {
            const int rr = e / RK;
            if (m0 + rr >= M) continue;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s += s_xl1[w * ROWS * RK + e];
            xl1[(m0 + rr) * RK + (e % RK)] = s;
        }
    }
}

}  // namespace

size_t act_quant_smem_bytes(int64_t K, int rank) {
    const int64_t G = K / 64;
    return sizeof(float) * (K + (ROWS * G + 1) / 2 + (size_t)waves_for(rank / 16) * ROWS * rank);
}

namespace {

template <int RT, int FMT, int CHT>
void launch_one(dim3 grid, size_t smem, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K,
                int64_t ldx, const float* inv_lambda, const uint16_t* l1t, uint8_t* qx, uint16_t* sx,
                float* xl1)
{
    if (smem > 65536)
        (void)hipFuncSetAttribute((const void*)act_quant_kernel<RT, FMT, CHT>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL((act_quant_kernel<RT, FMT, CHT>), grid, dim3(waves_for(RT) * 64), smem, stream,
                       x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1);
}

template <int FMT>
hipError_t launch_fmt(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                      const float* inv_lambda, const uint16_t* l1t, int rank,
                      uint8_t* qx, uint16_t* sx, float* xl1, hipStream_t stream)
{
    const dim3 grid((unsigned)((M + ROWS - 1) / ROWS));
    const size_t smem = act_quant_smem_bytes(K, rank);
    switch (rank / 16) {
    // the MXFP4 form with 16 waves and at least 8 groups per wave (K >= 8192)
    // runs faster with four groups in flight; the INT4 form does not
#define CASE(RTV) case RTV: \
        if constexpr (FMT == 1 && waves_for(RTV) == 16) { \
            if (K >= 8192) { \
                launch_one<RTV, FMT, 4>(grid, smem, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); \
                break; \
            } \
        } \
        launch_one<RTV, FMT, 0>(grid, smem, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
        CASE(0) CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            const float* inv_lambda, const uint16_t* l1t, int rank,
                            uint8_t* qx, uint16_t* sx, float* xl1, hipStream_t stream)
{
    return launch_fmt<0>(x, M, K, ldx, inv_lambda, l1t, rank, qx, sx, xl1, stream);
}

hipError_t launch_act_quant_mxfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const float* inv_lambda, const uint16_t* l1t, int rank,
                                  uint8_t* qx, uint8_t* sx, float* xl1, hipStream_t stream)
{
    return launch_fmt<1>(x, M, K, ldx, inv_lambda, l1t, rank, qx, (uint16_t*)sx, xl1, stream);
}
