// svdq_gemm_w4a4 kernel: 4-bit x 4-bit group GEMM with per-group fp16 scales,
// the low-rank up-projection and bias in the epilogue (optional GELU).
//
// The pages attribute to the original engine a fusion of the low-rank
// up-projection with the 4-bit matmul (remio.ai page, section "SVDQuant moves
// hard values out of 4-bit"). The CDNA4 design:
//  - INT4 codes in [-7, 7] are exact FP8 E4M3 values, so one
//    v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) forms one 64-wide
//    group's integer partial P_g exactly in fp32 (no int->float conversion);
//  - the two-sided scale S = sx (x) sw of a 32x32 block is an outer product;
//    a v_mfma_f32_32x32x16_f16 with a single non-zero k forms it exactly
//    (fp16 x fp16 fits fp32), so the matrix pipe, not the VALU, builds it and
//    the VALU does one FMA per output element per group: acc += P_g * S_g;
//  - packed nibbles are expanded to FP8 once per workgroup while a group is
//    staged into LDS, in MFMA lane order, so each wave reads a 32x64 operand
//    fragment as one conflict-free 2 KB block; raw packed data is prefetched
//    three groups ahead in registers;
//  - block tile 256 x 192 (8 waves of 64 x 96): the QKV shape (4096 x 9216)
//    is 768 tiles = 3 per CU; tiles are swizzled so each XCD (own L2) works
//    on whole rows of tiles and shares their activation blocks;
//  - the accumulator starts from X_hat L1 L2 (bf16 MFMA on the hi/lo split of
//    the fp32 xl1); bias and GELU run in fp32 before the single rounding of
//    the output, which leaves through LDS as row-contiguous 16-byte stores.
#include "common.h"

namespace {

constexpr int BM = 256, BN = 192;
constexpr int WGM = 4, WGN = 2;              // wave grid
constexpr int TM = 2, TN = 3;                // 32x32 blocks per wave
constexpr int NT = 512;
constexpr int FRAG_DW = 8;                   // a 32x64 fp8 fragment: 8 dwords per lane
constexpr int A_DW = (BM / 32) * 64 * FRAG_DW;
constexpr int B_DW = (BN / 32) * 64 * FRAG_DW;
constexpr int STAGE_BYTES = 4 * (A_DW + B_DW) + 2 * (BM + BN);
constexpr int OUT_LD = BN + 8;               // bf16 elements per LDS output row
constexpr int OUT_BYTES = BM * OUT_LD * 2;
constexpr int SMEM_BYTES = (2 * STAGE_BYTES > OUT_BYTES) ? 2 * STAGE_BYTES : OUT_BYTES;

DEV int out_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

struct Raw {
    uint4 a, b;
    uint32_t sa, sb;
};

struct Stage {
    uint32_t* A;
    uint32_t* B;
    uint16_t* SA;
    uint16_t* SB;
};

DEV Stage stage_ptr(char* smem, int s) {
    char* base = smem + s * STAGE_BYTES;
    Stage st;
    st.A = (uint32_t*)base;
    st.B = st.A + A_DW;
    st.SA = (uint16_t*)(st.B + B_DW);
    st.SB = st.SA + BM;
    return st;
}

// Per-thread staging sources: thread t stages row t/2, half t%2 of the A tile
// (all 512 threads) and of the B tile (t < 2 * BN). Rows past the end are
// clamped to the last row: what they load only reaches output rows/columns
// that are never stored.
struct Src {
    const uint8_t* a;
    const uint8_t* b;
    const uint16_t* sa;
    const uint16_t* sb;
};

template <bool SCALES>
DEV void load_raw(Raw& r, const Src& src, int g) {
    r.a = *(const uint4*)(src.a + (int64_t)g * 32);
    r.b = *(const uint4*)(src.b + (int64_t)g * 32);
    if constexpr (SCALES) {
        r.sa = src.sa[g];
        r.sb = src.sb[g];
    } else {
        r.sa = 0u;
        r.sb = 0u;
    }
}

DEV void expand_store(const uint4& raw, uint32_t* __restrict__ tile, int rr, int half) {
    uint32_t o[8];
    int4sm_to_fp8(raw.x, o[0], o[1]);
    int4sm_to_fp8(raw.y, o[2], o[3]);
    int4sm_to_fp8(raw.z, o[4], o[5]);
    int4sm_to_fp8(raw.w, o[6], o[7]);
    uint32_t* dst = tile + ((rr >> 5) * 64 + (rr & 31) + 32 * half) * FRAG_DW;
    *(uint4*)(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(dst + 4) = make_uint4(o[4], o[5], o[6], o[7]);
}

DEV void store_raw(const Raw& r, const Stage& st, int tid) {
    const int rr = tid >> 1, half = tid & 1;
    expand_store(r.a, st.A, rr, half);
    if (half == 0) st.SA[rr] = (uint16_t)r.sa;
    if (rr < BN) {
        expand_store(r.b, st.B, rr, half);
        if (half == 0) st.SB[rr] = (uint16_t)r.sb;
    }
}

DEV v8i read_frag(const uint32_t* __restrict__ tile, int blk, int lane) {
    const uint32_t* src = tile + (blk * 64 + lane) * FRAG_DW;
    const uint4 a = *(const uint4*)src, b = *(const uint4*)(src + 4);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Operand of the outer-product MFMA: only k = 0 (element 0 of lanes 0..31) is
// non-zero; A and B share the k layout, so the product is s_row * s_col.
DEV v8h scale_operand(uint16_t s, int lane) {
    const uint32_t v = (lane < 32) ? (uint32_t)s : 0u;
    return __builtin_bit_cast(v8h, make_uint4(v, 0u, 0u, 0u));
}

template <int MODE, int ACT>   // MODE 0: bf16 out, 1: fp32 out, 2: integer partials dump
__global__ __launch_bounds__(NT, 1) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    const float* __restrict__ xl1, const uint16_t* __restrict__ l2t, int rank,
    const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int64_t M, int64_t N, int64_t K,
    int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* __restrict__ part)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // tile index, swizzled so that consecutive blocks on one XCD (blocks are
    // dealt round-robin to the 8 XCDs) walk along one row of tiles
    const int64_t mext = (MODE == 2) ? pmc : M, next = (MODE == 2) ? pnc : N;
    const int tiles_n = (int)((next + BN - 1) / BN);
    const int tiles = tiles_n * (int)((mext + BM - 1) / BM);
    int t = blockIdx.x;
    if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
    const int64_t m0 = (MODE == 2 ? pm0 : 0) + (int64_t)(t / tiles_n) * BM;
    const int64_t n0 = (MODE == 2 ? pn0 : 0) + (int64_t)(t % tiles_n) * BN;
    const int64_t mlim = (MODE == 2) ? pm0 + pmc : M;
    const int64_t nlim = (MODE == 2) ? pn0 + pnc : N;
    const int G = (int)(K / 64);

    Src src;
    {
        const int rr = tid >> 1, half = tid & 1;
        const int64_t ra = (m0 + rr < mlim) ? m0 + rr : mlim - 1;
        const int64_t rb = (n0 + (rr % BN) < nlim) ? n0 + (rr % BN) : nlim - 1;
        src.a = qx + ra * (K / 2) + 16 * half;
        src.b = qw + rb * (K / 2) + 16 * half;
        src.sa = (MODE != 2) ? sx + ra * G : nullptr;
        src.sb = (MODE != 2) ? sw + rb * G : nullptr;
    }

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    constexpr bool SC = (MODE != 2);
    Raw r0, r1, r2;
    // group indices past the end are clamped to the last group: the extra
    // loads are harmless and keep the pipeline free of branches
    load_raw<SC>(r0, src, 0);
    load_raw<SC>(r1, src, G > 1 ? 1 : G - 1);
    load_raw<SC>(r2, src, G > 2 ? 2 : G - 1);

    // low-rank branch while the first groups are in flight: acc = xl1 L2
    if (MODE != 2 && rank > 0) {
        const int h = lane >> 5;
        for (int ks = 0; ks < rank / 16; ++ks) {
            v8bf ah[TM], al[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                int64_t row = m0 + wm * 32 * TM + i * 32 + (lane & 31);
                row = row < M ? row : M - 1;
                const float4 u0 = *(const float4*)(xl1 + row * rank + ks * 16 + 8 * h);
                const float4 u1 = *(const float4*)(xl1 + row * rank + ks * 16 + 8 * h + 4);
                const float xv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const __bf16 hb = (__bf16)xv[jj];
                    ah[i][jj] = hb;
                    al[i][jj] = (__bf16)(xv[jj] - (float)hb);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
                col = col < N ? col : N - 1;
                b[j] = *(const v8bf*)(l2t + col * rank + ks * 16 + 8 * h);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j] = mfma_bf16_32x32x16(ah[i], b[j], acc[i][j]);
                    acc[i][j] = mfma_bf16_32x32x16(al[i], b[j], acc[i][j]);
                }
        }
    }

    store_raw(r0, stage_ptr(smem, 0), tid);
    __syncthreads();

    const v16f zero = {};
    // One group: stage g+1 from its registers, refill them with group g+3,
    // then run the MFMAs of group g from LDS stage g%2.
    auto step = [&](int g, Raw& rn, Raw& rfill) {
        store_raw(rn, stage_ptr(smem, (g + 1) & 1), tid);
        load_raw<SC>(rfill, src, (g + 3 < G) ? g + 3 : G - 1);
        const Stage st = stage_ptr(smem, g & 1);
        v8i a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = read_frag(st.A, wm * TM + i, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = read_frag(st.B, wn * TN + j, lane);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const v8h so = scale_operand(st.SA[wm * 32 * TM + i * 32 + (lane & 31)], lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                // one 32x32 block in flight per wave keeps P and S within the
                // register budget of two waves per SIMD; the other wave on the
                // SIMD overlaps its MFMAs with this wave's FMAs
                __builtin_amdgcn_sched_barrier(0);
                const v16f p = mfma_f8_32x32x64(a[i], b[j], zero);
                if constexpr (MODE == 2) {
                    const int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int64_t row = m0 + wm * 32 * TM + i * 32 + out_row(e, lane);
                        if (row < mlim && col < nlim)
                            part[((row - pm0) * pnc + (col - pn0)) * G + g] = (int32_t)p[e];
                    }
                } else {
                    const v8h wo = scale_operand(st.SB[wn * 32 * TN + j * 32 + (lane & 31)], lane);
                    const v16f s = mfma_f16_32x32x16(so, wo, zero);
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(p[e], s[e], acc[i][j][e]);
                }
            }
        }
        __syncthreads();
    };

    for (int g = 0; g < G; g += 3) {
        step(g, r1, r0);
        if (g + 1 < G) step(g + 1, r2, r1);
        if (g + 2 < G) step(g + 2, r0, r2);
    }

    if constexpr (MODE == 0) {
        // bias, GELU, bf16 rounding; transpose through LDS for row-contiguous stores
        uint16_t* out = (uint16_t*)smem;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int lc = wn * 32 * TN + j * 32 + (lane & 31);
            const int64_t col = n0 + lc;
            const float bv = (bias && col < N) ? bf16_lo_to_f32(bias[col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = acc[i][j][e] + bv;
                    if constexpr (ACT == 1) v = gelu_tanh_f32(v);
                    const int lr = wm * 32 * TM + i * 32 + out_row(e, lane);
                    out[lr * OUT_LD + lc] = f32_to_bf16_bits(v);
                }
        }
        __syncthreads();
        constexpr int CHUNKS = BN / 8;              // 16-byte chunks per tile row
        for (int c = tid; c < BM * CHUNKS; c += NT) {
            const int lr = c / CHUNKS, lc = (c % CHUNKS) * 8;
            const int64_t row = m0 + lr, col = n0 + lc;
            if (row < M && col < N)
                *(uint4*)((uint16_t*)y + row * ldy + col) = *(const uint4*)(out + lr * OUT_LD + lc);
        }
    } else if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
            if (col >= N) continue;
            const float bv = bias ? bf16_lo_to_f32(bias[col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * 32 * TM + i * 32 + out_row(e, lane);
                    if (row >= M) continue;
                    float v = acc[i][j][e] + bv;
                    if constexpr (ACT == 1) v = gelu_tanh_f32(v);
                    ((float*)y)[row * ldy + col] = v;
                }
        }
    }
}

template <int MODE, int ACT>
void launch_mode(dim3 grid, hipStream_t stream, const uint8_t* qx, const uint16_t* sx,
                 const uint8_t* qw, const uint16_t* sw, const float* xl1, const uint16_t* l2t,
                 int rank, const uint16_t* bias, void* y, int64_t ldy, int64_t M, int64_t N,
                 int64_t K, int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* p) {
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)gemm_w4a4_kernel<MODE, ACT>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
        attr = true;
    }
    hipLaunchKernelGGL((gemm_w4a4_kernel<MODE, ACT>), grid, dim3(NT), SMEM_BYTES, stream, qx, sx,
                       qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, pm0, pmc, pn0, pnc, p);
}

}  // namespace

hipError_t launch_gemm_w4a4(const uint8_t* qx, const uint16_t* sx, const uint8_t* qw,
                            const uint16_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                            const uint16_t* bias, int act, void* y, int y_f32, int64_t ldy,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const int64_t tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    const dim3 grid((unsigned)tiles);
    if (y_f32) {
        if (act) launch_mode<1, 1>(grid, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
        else launch_mode<1, 0>(grid, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
    } else {
        if (act) launch_mode<0, 1>(grid, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
        else launch_mode<0, 0>(grid, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4_partials(const uint8_t* qx, const uint8_t* qw, int64_t M, int64_t N,
                                     int64_t K, int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                     int32_t* p, hipStream_t stream)
{
    const int64_t tiles = ((nc + BN - 1) / BN) * ((mc + BM - 1) / BM);
    launch_mode<2, 0>(dim3((unsigned)tiles), stream, qx, nullptr, qw, nullptr, nullptr, nullptr, 0,
                      nullptr, nullptr, 0, M, N, K, m0, mc, n0, nc, p);
    return hipGetLastError();
}
