// svdq_quantize_act kernel: smoothing + rank-r down-projection + symmetric
// INT4 group-64 quantisation of the activations, in one pass over X.
//
// The fusion of the low-rank down-projection with input quantisation is the
// one the remio.ai page attributes to the original Nunchaku engine (section
// "SVDQuant moves hard values out of 4-bit"); here it is re-derived for CDNA4:
//  - one workgroup owns 16 token rows; its waves take the 64-wide groups of
//    K round-robin, so every row is read from HBM exactly once with 128-byte
//    contiguous row segments per group; in this register form (8 waves) each
//    wave issues the loads of six of its groups at once (and the L1
//    fragments one group ahead) before it quantises them;
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
// Ranks up to 32 run the LDS-staged form further down (same arithmetic, the
// loads of X staged through LDS); this register form serves ranks 48-128.
// The MXFP4 form (FMT 1) shares all of this and differs in the per-value
// step: a 32-value block spans two lanes (l, l ^ 16); its E8M0 exponent is
// floor(log2(amax)) - 2 clamped to [-127, 127], read off the exponent field
// of amax; each value is scaled by the exact power of two 2^-e and rounded to
// the nearest E2M1 value (ties to mantissa 0, saturating at 6) by
// v_cvt_scalef32_pk_fp4_f32 with scale 1 (OCP Microscaling Formats v1.0:
// E2M1, E8M0, conversion from FP32). The instruction keeps the sign of values
// that round to zero; those nibbles get sign 0 afterwards.
#include "common.h"
#include "int4_fields.h"

namespace {

constexpr int ROWS = 16;

// RT = rank / 16 (3..8 here); FMT 0: INT4 g64, 1: MXFP4; CHT: groups each
// wave keeps in flight (0: six); WV: waves per workgroup
template <int RT, int FMT, int CHT, int WV>
__global__ __launch_bounds__(WV * 64) void act_quant_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ inv_lambda, const uint16_t* __restrict__ l1t,
    uint8_t* __restrict__ qx, uint16_t* __restrict__ sx, float* __restrict__ xl1)
{
    constexpr int RTX = RT > 0 ? RT : 1;
    constexpr int WAVES = WV, NTH = WAVES * 64;
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

            const uint2 word = codes16_fp6(v, inv);
            if (valid) {
                *(uint2*)(qx + row * (K / 2) + g * 32 + 8 * p) = word;
                if (p == 0) s_sx[r * G + g] = __builtin_bit_cast(uint16_t, s16);
            }
        } else {
            // block 2g + (p >> 1) of the row; e = floor(log2 amax) - 2 from the
            // exponent field (a zero or subnormal amax clamps to -127)
            const int e = mx_block_exponent(amax);
            const float sc = mx_inv_scale(e);                              // 2^-e, exact
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
    constexpr int CH = CHT ? CHT : 6;
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

// ---- the LDS-staged form (ranks up to 32) ---------------------------------
// Same per-value steps and the same group-to-wave assignment, but a wave's
// X rows and smoothing reciprocals travel from memory straight into LDS
// (buffer_load ... lds), into a ring of NS slots per wave, one group per
// slot: a wave requests NS groups at once at its start without holding any
// of them in registers, needs no workgroup barrier before its first group
// (each wave loads the reciprocals of its own groups), and reads a slot as
// soon as that slot's loads have landed (the slots are separate LDS objects,
// so the compiler's wait before a slot's reads covers only the loads issued
// up to that slot's).

typedef __attribute__((address_space(3))) void lds_void;

// 16 (or 4) bytes per lane from global memory into LDS at lds + 16 (4) * lane
DEV void dma16(rsrc_t r, char* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
DEV void dma4(rsrc_t r, char* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
}

// one group of one wave: 16 rows x 128 bytes of X (16-byte chunk c of row
// r at r * 128 + 16 * (c ^ ((r / 2) % 8)), so the 16 lanes that read one
// chunk column of the 16 rows hit distinct banks), then 64 fp32 reciprocals
constexpr int SLOT = ROWS * 128 + 256;

template <int V> struct IC { static constexpr int value = V; };
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int RT, int FMT, int WV, int NS, bool SM>
__global__ __launch_bounds__(WV * 64) void act_quant_lds_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ inv_lambda, const uint16_t* __restrict__ l1t,
    uint8_t* __restrict__ qx, uint16_t* __restrict__ sx, float* __restrict__ xl1)
{
    static_assert(RT <= 2 && NS >= 1 && NS <= 6, "rank <= 32 (the partials reuse slot 0), 1..6 slots");
    constexpr int RTX = RT > 0 ? RT : 1;
    constexpr int NTH = WV * 64;
    __shared__ __attribute__((aligned(16))) char xs0[WV * SLOT];
    __shared__ __attribute__((aligned(16))) char xs1[NS > 1 ? WV * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char xs2[NS > 2 ? WV * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char xs3[NS > 3 ? WV * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char xs4[NS > 4 ? WV * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char xs5[NS > 5 ? WV * SLOT : 16];
    auto slot_of = [&](auto S) -> char* {
        constexpr int s = decltype(S)::value;
        if constexpr (s == 0) return xs0;
        else if constexpr (s == 1) return xs1;
        else if constexpr (s == 2) return xs2;
        else if constexpr (s == 3) return xs3;
        else if constexpr (s == 4) return xs4;
        else return xs5;
    };
    // calls f(IC<0>), ..., f(IC<NS - 1>) in order
    auto each_slot = [&](auto&& f) __attribute__((always_inline)) {
        f(IC<0>{});
        if constexpr (NS > 1) f(IC<1>{});
        if constexpr (NS > 2) f(IC<2>{});
        if constexpr (NS > 3) f(IC<3>{});
        if constexpr (NS > 4) f(IC<4>{});
        if constexpr (NS > 5) f(IC<5>{});
    };

    const int G = (int)(K / 64), G4 = (G + 3) / 4;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t m0 = (int64_t)blockIdx.x * ROWS;
    const int rows_here = (int)(M - m0 < ROWS ? M - m0 : ROWS);
    const int r = lane & 15, p = lane >> 4;
    const int64_t row = m0 + r;
    const bool valid = r < rows_here;
    const int n = (G > wave) ? (G - wave + WV - 1) / WV : 0;
    auto gidx = [&](int i) { const int gi = wave + WV * i; return gi < G ? gi : G - 1; };

    // X of the block's rows: rows past the end fall outside the buffer and
    // read 0 (nothing of theirs is stored); byte offsets fit in 31 bits
    // (16 ldx < 2^30, checked on the host)
    const rsrc_t rx = make_rsrc(x + m0 * ldx, (int64_t)rows_here * ldx * 2);
    const rsrc_t ri = make_rsrc(inv_lambda, SM ? K * 4 : 0);
    const int xr0 = lane >> 3, xr1 = 8 + (lane >> 3);
    const int vx0 = xr0 * (int)ldx * 2 + 16 * ((lane & 7) ^ ((xr0 >> 1) & 7));
    const int vx1 = xr1 * (int)ldx * 2 + 16 * ((lane & 7) ^ ((xr1 >> 1) & 7));

    v4f acc[RTX];
#pragma unroll
    for (int t = 0; t < RTX; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    v8bf lv[NS][RTX][2];

    auto issue = [&](auto S, int i) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        const int g = gidx(i);
        char* base = slot_of(S) + wave * SLOT;
        dma16(rx, base, vx0, g * 128);
        dma16(rx, base + 1024, vx1, g * 128);
        if constexpr (SM) dma4(ri, base + ROWS * 128, 4 * lane, g * 256);
        if constexpr (RT > 0) {
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const uint16_t* lf = l1t + ((int64_t)(g * RT + t) * 2) * 512 + lane * 8;
                lv[s][t][0] = *(const v8bf*)(lf);
                lv[s][t][1] = *(const v8bf*)(lf + 512);
            }
        }
    };

    // Stores go through buffer descriptors whose range check drops the rows
    // past M and the lanes with nothing to store (offset past the end), so
    // the group loop has no branches: the compiler's waits for a slot then
    // count exactly the loads issued after that slot's.
    const rsrc_t rq = make_rsrc(qx + m0 * (K / 2), (int64_t)rows_here * (K / 2));
    const int vq = valid ? r * (int)(K / 2) + 8 * p : INT32_MAX;
    constexpr int OFF = INT32_MAX;      // outside every descriptor here
    auto process = [&](auto S, int i) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        const int g = gidx(i);
        const char* base = slot_of(S) + wave * SLOT;
        const int sw = (r >> 1) & 7;
        const uint4 xa = *(const uint4*)(base + r * 128 + 16 * ((2 * p) ^ sw));
        const uint4 xb = *(const uint4*)(base + r * 128 + 16 * ((2 * p + 1) ^ sw));
        const uint32_t w[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        float v[16];
        if constexpr (SM) {
            const float4* ip = (const float4*)(base + ROWS * 128 + 64 * p);
            const float4 i0 = ip[0], i1 = ip[1], i2 = ip[2], i3 = ip[3];
            const float iv[16] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w,
                                  i2.x, i2.y, i2.z, i2.w, i3.x, i3.y, i3.z, i3.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[2 * j] = bf16_lo_to_f32(w[j]) * iv[2 * j];
                v[2 * j + 1] = bf16_hi_to_f32(w[j]) * iv[2 * j + 1];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[2 * j] = bf16_lo_to_f32(w[j]);
                v[2 * j + 1] = bf16_hi_to_f32(w[j]);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        // the records of this group's quad for the block's rows: [G4][M][8 bytes]
        const rsrc_t rs = make_rsrc((const uint8_t*)sx + ((int64_t)(g >> 2) * M + m0) * 8, (int64_t)rows_here * 8);
        if constexpr (FMT == 0) {
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const float s32 = fminf(amax / 7.0f, 65504.0f);
            const _Float16 s16 = (_Float16)s32;
            const float sf = (float)s16;
            const float inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;
            const uint2 word = codes16_fp6(v, inv);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{word.x, word.y}, rq, vq, g * 32, 0);
            // lane p = 0 of each row stores the group's fp16 scale
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, s16), rs,
                                                  p == 0 ? r * 8 + 2 * (g & 3) : OFF, 0, 0);
        } else {
            const int e = mx_block_exponent(amax);
            const float sc = mx_inv_scale(e);
            float t[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) t[j] = v[j] * sc;
            const uint2 word = make_uint2(e2m1_x8(t), e2m1_x8(t + 8));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{word.x, word.y}, rq, vq, g * 32, 0);
            // lanes p = 0, 2 store the exponents of blocks 2g, 2g + 1 at
            // bytes (g % 4) and 4 + (g % 4) of the row's record
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(e + 127), rs,
                                                 (p & 1) == 0 ? r * 8 + 4 * (p >> 1) + (g & 3) : OFF, 0, 0);
        }

        if constexpr (RT > 0) {
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
                acc[t] = mfma_bf16_16x16x32(ah0, lv[s][t][0], acc[t]);
                acc[t] = mfma_bf16_16x16x32(al0, lv[s][t][0], acc[t]);
                acc[t] = mfma_bf16_16x16x32(ah1, lv[s][t][1], acc[t]);
                acc[t] = mfma_bf16_16x16x32(al1, lv[s][t][1], acc[t]);
            }
        }
    };

    // Ring of NS slots: group i lives in slot i % NS. The first NS groups are
    // requested unconditionally (a wave with fewer groups requests copies of
    // the last one, never read); the steady loop refills each slot as soon as
    // its group is read, and every refill there is needed, so no path through
    // the loop issues fewer loads than another; the last groups run after it.
    each_slot([&](auto S) __attribute__((always_inline)) { issue(S, decltype(S)::value); });
    int c0 = 0;
    // (the scheduling barriers keep one group's work from being interleaved
    // with the next group's, which would only raise register pressure)
    for (; c0 + 2 * NS <= n; c0 += NS)
        each_slot([&](auto S) __attribute__((always_inline)) {
            process(S, c0 + decltype(S)::value);
            issue(S, c0 + decltype(S)::value + NS);
            __builtin_amdgcn_sched_barrier(0);
        });
    auto last = [&](auto S) __attribute__((always_inline)) {
        const int i = c0 + decltype(S)::value;
        if (i < n) {
            process(S, i);
            if (i + NS < n) issue(S, i + NS);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    each_slot(last);
    c0 += NS;
    each_slot(last);

    // the last quad's records hold zeros for the groups past the end of K
    if (wave == WV - 1 && G % 4 != 0) {
        uint8_t* rec0 = (uint8_t*)sx + ((int64_t)(G4 - 1) * M + m0) * 8;
        for (int e = lane; e < ROWS * 8; e += 64) {
            const int rr = e / 8, b = e % 8;
            const int gg = 4 * (G4 - 1) + (FMT == 0 ? b / 2 : b % 4);
            if (rr < rows_here && gg >= G) rec0[e] = 0;
        }
    }

    if constexpr (RT > 0) {
        // per-wave partials in the wave's own part of slot 0 (its last use of
        // that part is behind it), then summed over the waves in a fixed order
        const int RK = 16 * RT;
        float* part = (float*)(xs0 + wave * SLOT);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[(4 * p + i) * RK + 16 * t + r] = acc[t][i];
        __syncthreads();
        for (int e = tid; e < ROWS * RK; e += NTH) {
            const int rr = e / RK;
            if (rr >= rows_here) continue;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WV; ++w) s += ((const float*)(xs0 + w * SLOT))[e];
            xl1[(m0 + rr) * RK + (e % RK)] = s;
        }
    }
}

}  // namespace

// LDS of a register-form launch with `waves` waves
size_t act_quant_smem_bytes_w(int64_t K, int rank, int waves) {
    const int64_t G = K / 64;
    return sizeof(float) * (K + (ROWS * G + 1) / 2 + (size_t)waves * ROWS * rank);
}

// LDS a launch of (K, rank) needs: the LDS-staged form (ranks up to 32)
// uses a fixed amount, at most 16 waves x 3 slots; the register form (8
// waves) holds K reciprocals and the per-wave partials
size_t act_quant_smem_bytes(int64_t K, int rank) {
    return rank <= 32 ? (size_t)16 * 3 * SLOT : act_quant_smem_bytes_w(K, rank, 8);
}

namespace {

template <int RT, int FMT, int CHT, int WV>
void launch_one(dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K,
                int64_t ldx, const float* inv_lambda, const uint16_t* l1t, uint8_t* qx, uint16_t* sx,
                float* xl1)
{
    const size_t smem = act_quant_smem_bytes_w(K, RT * 16, WV);
    if (smem > 65536)
        (void)hipFuncSetAttribute((const void*)act_quant_kernel<RT, FMT, CHT, WV>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL((act_quant_kernel<RT, FMT, CHT, WV>), grid, dim3(WV * 64), smem, stream,
                       x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1);
}

template <int RT, int FMT, int WV, int NS>
void launch_lds(dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                const float* inv_lambda, const uint16_t* l1t, uint8_t* qx, uint16_t* sx, float* xl1)
{
    if (inv_lambda)
        hipLaunchKernelGGL((act_quant_lds_kernel<RT, FMT, WV, NS, true>), grid, dim3(WV * 64), 0, stream,
                           x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1);
    else
        hipLaunchKernelGGL((act_quant_lds_kernel<RT, FMT, WV, NS, false>), grid, dim3(WV * 64), 0, stream,
                           x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1);
}

// LDS-staged form, (waves, slots per wave): 0 = (16, 2), 1 = (16, 3),
// 2 = (8, 3); LDS 73.7, 110.6 and 55.3 KB. Chosen from timings over 12
// rotated copies of X, rank 32 (INT4 / MXFP4; register form for reference):
// 4096 x 3072: register 13.6 / 12.5 us, (16, 3) 11.6 / spills, (8, 3) 12.0
// / 11.0; 4608 x 3072 (more row blocks than CUs): register 20.3 / 19.5 us,
// (8, 3) 18.5 / 18.3; 4608 x 12288: register 73.7 / 71.0 us, (16, 2) 65.7 /
// 63.7.
template <int FMT>
int lds_config(bool shared_cu, int64_t K) {
    if (K >= 8192) return 0;
    if (FMT == 1 || shared_cu) return 2;
    return 1;
}

template <int RT, int FMT>
void launch_lds_rank(int cfg, dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K,
                     int64_t ldx, const float* inv_lambda, const uint16_t* l1t, uint8_t* qx, uint16_t* sx,
                     float* xl1)
{
    switch (cfg) {
    case 0: launch_lds<RT, FMT, 16, 2>(grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
    case 1:
        if constexpr (FMT == 0) {      // the MXFP4 kernel spills in this shape; it takes (8, 3)
            launch_lds<RT, FMT, 16, 3>(grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1);
            break;
        }
        [[fallthrough]];
    default: launch_lds<RT, FMT, 8, 3>(grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
    }
}

template <int FMT>
hipError_t launch_fmt(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                      const float* inv_lambda, const uint16_t* l1t, int rank,
                      uint8_t* qx, uint16_t* sx, float* xl1, int cus, hipStream_t stream)
{
    const int64_t blocks = (M + ROWS - 1) / ROWS;
    const dim3 grid((unsigned)blocks);
    const bool shared_cu = blocks > cus;          // more row blocks than CUs: (8, 3), two workgroups per CU
    // ranks up to 32 with 16 rows of X addressable by 31-bit byte offsets
    if (rank <= 32) {
        const int cfg = lds_config<FMT>(shared_cu, K);
        switch (rank / 16) {
        case 0: launch_lds_rank<0, FMT>(cfg, grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
        case 1: launch_lds_rank<1, FMT>(cfg, grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
        default: launch_lds_rank<2, FMT>(cfg, grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
        }
        return hipGetLastError();
    }
    // ranks 48-128: the register form, 8 waves with six groups in flight each
    switch (rank / 16) {
#define CASE(RTV) case RTV: \
        launch_one<RTV, FMT, 0, 8>(grid, stream, x, M, K, ldx, inv_lambda, l1t, qx, sx, xl1); break;
        CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            const float* inv_lambda, const uint16_t* l1t, int rank,
                            uint8_t* qx, uint16_t* sx, float* xl1, int cus, hipStream_t stream)
{
    return launch_fmt<0>(x, M, K, ldx, inv_lambda, l1t, rank, qx, sx, xl1, cus, stream);
}

hipError_t launch_act_quant_mxfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const float* inv_lambda, const uint16_t* l1t, int rank,
                                  uint8_t* qx, uint8_t* sx, float* xl1, int cus, hipStream_t stream)
{
    return launch_fmt<1>(x, M, K, ldx, inv_lambda, l1t, rank, qx, (uint16_t*)sx, xl1, cus, stream);
}
