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
//    activations keep ~16 mantissa bits; hi/lo and the group sums are
//    prepared once per workgroup in LDS, already in MFMA operand order.
//  - A workgroup owns 64 output columns (4 waves x 16); each wave streams the
//    whole K of its columns, keeping the next batch of 16 groups (codes,
//    scales, zeros) in flight while it computes the current batch, so about
//    70 KB per CU is in flight: enough to cover HBM latency at full rate.
#include "common.h"

namespace {

constexpr int NT = 256;
constexpr int WAVES = 4;
constexpr int COLS = 16 * WAVES;
constexpr int BATCH = 16;         // groups per prefetch batch
constexpr int MAXM = 16;
constexpr int LDS_ELEMS = 32768;  // x~ elements (rows x K chunk) held in LDS, hi + lo

// K chunk held in LDS: a multiple of 2048 (32 groups, two prefetch batches),
// so every chunk starts on an even batch
__host__ __device__ inline int kchunk(int M, int64_t K) {
    const int kc = (LDS_ELEMS / M) & ~2047;
    return (int)(K < kc ? K : kc);
}

// MFMA slot j of a step holds element perm[j] of the lane's 8 codes, because
// the 8 nibbles of a dword are expanded as pairs (t, t + 4).
DEV int slot_of(int o) { return (o < 4) ? 2 * o : 2 * (o - 4) + 1; }

DEV v8bf codes_to_bf16(uint32_t x) {
    uint32_t d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) d[t] = ((x >> (4 * t)) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(v8bf, make_uint4(d[0], d[1], d[2], d[3]));
}

struct Batch {
    uint2 q[BATCH];
    uint32_t sz[BATCH];     // scale (low 16 bits) and zero (high 16 bits), fp16
};

__global__ __launch_bounds__(NT) void gemv_w4a16_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, const float* __restrict__ inv_s,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t N, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y)
{
    extern __shared__ uint32_t smem_u[];
    const int KC = kchunk(M, K);
    const int steps_c = KC / 32;
    // [2 (hi, lo)][steps][4 p][M][8 bf16]  then  xsum [KC/64][MAXM]
    uint16_t* s_a = (uint16_t*)smem_u;
    float* s_xsum = (float*)(smem_u + (2 * steps_c * 4 * M * 8) / 2);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, p = lane >> 4;
    const int64_t n = (int64_t)blockIdx.x * COLS + wave * 16 + c;
    const int64_t ncl = n < N ? n : N - 1;      // columns past N read the last one, never stored
    const int G = (int)(K / 64);
    const uint8_t* wrow = qw + ncl * (K / 2) + 8 * p;
    const uint16_t* srow = scale + ncl * G;
    const uint16_t* zrow = zero + ncl * G;

    auto load_batch = [&](Batch& b, int g0) {
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int g = (g0 + i < G) ? g0 + i : G - 1;     // clamped: stays in bounds
            b.q[i] = *(const uint2*)(wrow + (int64_t)g * 32);
            b.sz[i] = (uint32_t)srow[g] | ((uint32_t)zrow[g] << 16);
        }
    };

    v4f acc = {0.f, 0.f, 0.f, 0.f};
    Batch b0, b1;
    load_batch(b0, 0);

    for (int64_t k0 = 0; k0 < K; k0 += KC) {
        const int kc = (int)((K - k0) < KC ? (K - k0) : KC);
        const int gc = kc / 64, gbase = (int)(k0 / 64);
        __syncthreads();   // previous chunk's LDS reads are done
        // x~ hi/lo in MFMA order; item = (row m, 8 consecutive k); the 8 items
        // of one (row, group) are 8 consecutive threads, which sum their part.
        // Items are taken 8 per thread at a time with all their loads issued
        // first, so the prep costs one memory latency per 8 items.
        const int nitems = M * (kc / 8);
        constexpr int IB = 8;
        for (int it0 = 0; it0 < nitems; it0 += IB * NT) {
            uint4 raw[IB];
            float4 sc0[IB], sc1[IB];
#pragma unroll
            for (int u = 0; u < IB; ++u) {
                const int itc = min(it0 + u * NT + tid, nitems - 1);      // clamped: in bounds
                const int m = itc / (kc / 8), kk = (itc % (kc / 8)) * 8;
                raw[u] = *(const uint4*)(x + (int64_t)m * K + k0 + kk);
                if (inv_s) {
                    sc0[u] = *(const float4*)(inv_s + k0 + kk);
                    sc1[u] = *(const float4*)(inv_s + k0 + kk + 4);
                } else {
                    sc0[u] = make_float4(1.f, 1.f, 1.f, 1.f);
                    sc1[u] = sc0[u];
                }
            }
#pragma unroll
            for (int u = 0; u < IB; ++u) {
                const int it = it0 + u * NT + tid;
                if (it0 + u * NT >= nitems) break;        // uniform across the workgroup
                const bool live = it < nitems;
                const int itc = live ? it : nitems - 1;
                const int m = itc / (kc / 8), kk = (itc % (kc / 8)) * 8;
                const int gl = kk / 64, pp = (kk % 64) / 16, ss = (kk % 16) / 8;
                const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
                const float is[8] = {sc0[u].x, sc0[u].y, sc0[u].z, sc0[u].w,
                                     sc1[u].x, sc1[u].y, sc1[u].z, sc1[u].w};
                uint16_t hi[8], lo[8];
                float part = 0.0f;
#pragma unroll
                for (int o = 0; o < 8; ++o) {
                    const float xv = ((o & 1) ? bf16_hi_to_f32(w[o >> 1]) : bf16_lo_to_f32(w[o >> 1]));
                    const float xt = xv * is[o];
                    const __bf16 h = (__bf16)xt;
                    const __bf16 l = (__bf16)(xt - (float)h);
                    hi[slot_of(o)] = __builtin_bit_cast(uint16_t, h);
                    lo[slot_of(o)] = __builtin_bit_cast(uint16_t, l);
                    part += (float)h + (float)l;
                }
                // items it .. it+7 (aligned) are one (row, group): fixed-order tree sum
                part += __shfl_xor(part, 1);
                part += __shfl_xor(part, 2);
                part += __shfl_xor(part, 4);
                if (live) {
                    const int base = (((gl * 2 + ss) * 4 + pp) * M + m) * 8;
                    *(uint4*)(s_a + base) = make_uint4(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16),
                                                       hi[4] | ((uint32_t)hi[5] << 16), hi[6] | ((uint32_t)hi[7] << 16));
                    *(uint4*)(s_a + steps_c * 4 * M * 8 + base) =
                        make_uint4(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16),
                                   lo[4] | ((uint32_t)lo[5] << 16), lo[6] | ((uint32_t)lo[7] << 16));
                    if ((it & 7) == 0) s_xsum[gl * MAXM + m] = part;
                }
            }
        }
        __syncthreads();

        auto compute = [&](const Batch& cur, int g0) {
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int gl = g0 + i;
                if (gl >= gc) break;
                v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const v8bf bq = codes_to_bf16(st ? cur.q[i].y : cur.q[i].x);
                    v8bf ah, al;
                    if (c < M) {
                        const int base = (((gl * 2 + st) * 4 + p) * M + c) * 8;
                        ah = *(const v8bf*)(s_a + base);
                        al = *(const v8bf*)(s_a + steps_c * 4 * M * 8 + base);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) { ah[j] = (__bf16)0.0f; al[j] = (__bf16)0.0f; }
                    }
                    // A rows are activation rows (lane & 15), B columns are outputs
                    d = mfma_bf16_16x16x32(ah, bq, d);
                    d = mfma_bf16_16x16x32(al, bq, d);
                }
                const float sc = f16_bits_to_f32((uint16_t)(cur.sz[i] & 0xFFFFu));
                const float off = 128.0f + f16_bits_to_f32((uint16_t)(cur.sz[i] >> 16));
                const float4 xs = *(const float4*)(s_xsum + gl * MAXM + 4 * p);
                const float xsv[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float t = __builtin_fmaf(-off, xsv[e], d[e]);
                    acc[e] = __builtin_fmaf(sc, t, acc[e]);
                }
            }
        };
        // even batches live in b0, odd ones in b1; each load runs one batch ahead
        for (int g0 = 0; g0 < gc; g0 += 2 * BATCH) {
            load_batch(b1, gbase + g0 + BATCH);
            compute(b0, g0);
            load_batch(b0, gbase + g0 + 2 * BATCH);
            if (g0 + BATCH < gc) compute(b1, g0 + BATCH);
        }
    }

    // C layout (16x16): lane holds column c, rows 4p + e
    const float bv = bias ? bf16_lo_to_f32(bias[ncl]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * p + e;
        if (m < M && n < N) y[(int64_t)m * N + n] = f32_to_bf16_bits(acc[e] + bv);
    }
}

}  // namespace

size_t gemv_smem_bytes(int M, int64_t K) {
    const int KC = kchunk(M, K);
    return (size_t)2 * (KC / 32) * 4 * M * 8 * 2 + sizeof(float) * (KC / 64) * MAXM;
}

hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t K, const float* inv_s,
                             const uint8_t* qw, const uint16_t* scale, const uint16_t* zero,
                             int64_t N, const uint16_t* bias, uint16_t* y, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + COLS - 1) / COLS)), block(NT);
    const size_t smem = gemv_smem_bytes(M, K);
    if (smem > 65536)
        (void)hipFuncSetAttribute((const void*)gemv_w4a16_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL(gemv_w4a16_kernel, grid, block, smem, stream,
                       x, M, K, inv_s, qw, scale, zero, N, bias, y);
    return hipGetLastError();
}
