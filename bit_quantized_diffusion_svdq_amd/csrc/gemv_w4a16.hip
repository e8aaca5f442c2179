// awq_gemv_w4a16 kernel: 4-bit weights, 16-bit activations, few rows
// (adaLN / modulation projections; donmalab.com page, section on the two
// schemes). Memory-bound: the packed weights are streamed from HBM once and
// dequantised in registers.
//
// CDNA4 design:
//  - A nibble q becomes the bf16 value 128 + q exactly by OR-ing it into the
//    bf16 pattern of 128.0 (0x4300): one shift + one and-or per two codes.
//  - The bf16 MFMA (16x16x32) forms D_g = sum_k x~[m,k] (128 + q[n,k]) per
//    64-wide group; the zero point and the offset fold out through the
//    per-(row, group) sum of x~:  Y += s (D_g - (128 + z) sum_k x~).
//  - x~ = fp32(x) * inv_s is split into bf16 hi + lo (two MFMAs) so the
//    activations keep ~16 mantissa bits; hi/lo are prepared once per
//    workgroup in LDS, already in MFMA operand order.
//  - A workgroup owns 16 output columns; its 4 waves split the groups of K;
//    the 4 partial results are added in LDS in a fixed order.
#include "common.h"

namespace {

constexpr int NT = 256;
constexpr int KC = 1024;          // K chunk held in LDS
constexpr int MAXM = 16;

// MFMA slot j of a step holds element perm[j] of the lane's 8 codes, because
// the 8 nibbles of a dword are expanded as pairs (t, t + 4).
DEV int slot_of(int o) { return (o < 4) ? 2 * o : 2 * (o - 4) + 1; }

DEV void codes_to_bf16(uint32_t x, v8bf& b) {
    uint32_t d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) d[t] = ((x >> (4 * t)) & 0x000F000Fu) | 0x43004300u;
    b = __builtin_bit_cast(v8bf, make_uint4(d[0], d[1], d[2], d[3]));
}

__global__ __launch_bounds__(NT) void gemv_w4a16_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, const float* __restrict__ inv_s,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t N, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y)
{
    extern __shared__ uint32_t smem_u[];
    // [2 (hi, lo)][KC/32 steps][4 p][M][8 bf16]  +  xsum [M][KC/64]  + red [4][MAXM][16]
    uint16_t* s_a = (uint16_t*)smem_u;
    const int steps_c = KC / 32;
    float* s_xsum = (float*)(smem_u + (2 * steps_c * 4 * M * 8) / 2);
    float* s_red = s_xsum + M * (KC / 64);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, p = lane >> 4;
    const int64_t n = (int64_t)blockIdx.x * 16 + c;
    const int G = (int)(K / 64);
    const uint8_t* wrow = qw + n * (K / 2);

    v4f acc = {0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = 0; k0 < K; k0 += KC) {
        const int kc = (int)((K - k0) < KC ? (K - k0) : KC);
        const int gc = kc / 64;
        // issue this wave's weight, scale and zero loads for the chunk
        uint2 wq[KC / 64 / 4];
        float sc[KC / 64 / 4], zc[KC / 64 / 4];
#pragma unroll
        for (int i = 0; i < KC / 64 / 4; ++i) {
            const int gl = wave + 4 * i;
            if (gl < gc) {
                const int64_t g = k0 / 64 + gl;
                wq[i] = *(const uint2*)(wrow + g * 32 + 8 * p);
                sc[i] = f16_bits_to_f32(scale[n * G + g]);
                zc[i] = f16_bits_to_f32(zero[n * G + g]);
            }
        }
        __syncthreads();   // previous chunk's LDS reads are done
        // prepare x~ hi/lo in MFMA order: item = (row m, 8 consecutive k)
        for (int it = tid; it < M * (kc / 8); it += NT) {
            const int m = it / (kc / 8);
            const int kk = (it % (kc / 8)) * 8;          // offset inside the chunk
            const int gl = kk / 64, pp = (kk % 64) / 16, ss = (kk % 16) / 8;
            const uint4 raw = *(const uint4*)(x + (int64_t)m * K + k0 + kk);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                const float xv = ((o & 1) ? bf16_hi_to_f32(w[o >> 1]) : bf16_lo_to_f32(w[o >> 1]));
                const float xt = inv_s ? xv * inv_s[k0 + kk + o] : xv;
                const __bf16 h = (__bf16)xt;
                hi[slot_of(o)] = __builtin_bit_cast(uint16_t, h);
                lo[slot_of(o)] = f32_to_bf16_bits(xt - (float)h);
            }
            const int base = (((gl * 2 + ss) * 4 + pp) * M + m) * 8;
            uint4 vh, vl;
            vh.x = hi[0] | ((uint32_t)hi[1] << 16); vh.y = hi[2] | ((uint32_t)hi[3] << 16);
            vh.z = hi[4] | ((uint32_t)hi[5] << 16); vh.w = hi[6] | ((uint32_t)hi[7] << 16);
            vl.x = lo[0] | ((uint32_t)lo[1] << 16); vl.y = lo[2] | ((uint32_t)lo[3] << 16);
            vl.z = lo[4] | ((uint32_t)lo[5] << 16); vl.w = lo[6] | ((uint32_t)lo[7] << 16);
            *(uint4*)(s_a + base) = vh;
            *(uint4*)(s_a + steps_c * 4 * M * 8 + base) = vl;
        }
        __syncthreads();
        // per (row, group) sums of the split values, in a fixed order
        for (int it = tid; it < M * gc; it += NT) {
            const int m = it / gc, gl = it % gc;
            float sum = 0.0f;
            for (int st = 0; st < 2; ++st)
                for (int pp = 0; pp < 4; ++pp)
                    for (int j = 0; j < 8; ++j) {
                        const int idx = (((gl * 2 + st) * 4 + pp) * M + m) * 8 + j;
                        sum += bf16_lo_to_f32(s_a[idx]) + bf16_lo_to_f32(s_a[steps_c * 4 * M * 8 + idx]);
                    }
            s_xsum[m * (KC / 64) + gl] = sum;
        }
        __syncthreads();

#pragma unroll
        for (int i = 0; i < KC / 64 / 4; ++i) {
            const int gl = wave + 4 * i;
            if (gl >= gc) break;
            v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                v8bf b;
                codes_to_bf16(st ? wq[i].y : wq[i].x, b);
                v8bf ah, al;
                if (c < M) {
                    const int base = (((gl * 2 + st) * 4 + p) * M + c) * 8;
                    ah = *(const v8bf*)(s_a + base);
                    al = *(const v8bf*)(s_a + steps_c * 4 * M * 8 + base);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) { ah[j] = (__bf16)0.0f; al[j] = (__bf16)0.0f; }
                }
                // A operand rows are activation rows (lane & 15), B columns are outputs
                d = mfma_bf16_16x16x32(ah, b, d);
                d = mfma_bf16_16x16x32(al, b, d);
            }
            const float off = 128.0f + zc[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * p + e;
                const float xs = (m < M) ? s_xsum[m * (KC / 64) + gl] : 0.0f;
                const float t = __builtin_fmaf(-off, xs, d[e]);
                acc[e] = __builtin_fmaf(sc[i], t, acc[e]);
            }
        }
    }

    // C layout (16x16): lane holds column c, rows 4p + e
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[(wave * MAXM + 4 * p + e) * 16 + c] = acc[e];
    __syncthreads();
    if (tid < MAXM * 16) {
        const int m = tid / 16, cc = tid % 16;
        const int64_t nn = (int64_t)blockIdx.x * 16 + cc;
        if (m < M) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) v += s_red[(w * MAXM + m) * 16 + cc];
            if (bias) v += bf16_lo_to_f32(bias[nn]);
            y[(int64_t)m * N + nn] = f32_to_bf16_bits(v);
        }
    }
}

}  // namespace

size_t gemv_smem_bytes(int M) {
    return (size_t)2 * (KC / 32) * 4 * M * 8 * 2 + sizeof(float) * (M * (KC / 64) + 4 * MAXM * 16);
}

hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t K, const float* inv_s,
                             const uint8_t* qw, const uint16_t* scale, const uint16_t* zero,
                             int64_t N, const uint16_t* bias, uint16_t* y, hipStream_t stream)
{
    const dim3 grid((unsigned)(N / 16)), block(NT);
    const size_t smem = gemv_smem_bytes(M);
    if (smem > 65536)
        (void)hipFuncSetAttribute((const void*)gemv_w4a16_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL(gemv_w4a16_kernel, grid, block, smem, stream,
                       x, M, K, inv_s, qw, scale, zero, N, bias, y);
    return hipGetLastError();
}
