// svdq_gemm_w4a4 kernel: 4-bit x 4-bit group GEMM with per-group fp16 scales,
// the low-rank up-projection and bias in the epilogue (optional GELU).
//
// The pages attribute to the original engine a fusion of the low-rank
// up-projection with the 4-bit matmul (remio.ai page, section "SVDQuant moves
// hard values out of 4-bit"). The CDNA4 design:
//  - INT4 codes in [-7, 7] are exact FP8 E4M3 subnormals (q * 2^-9), and the
//    E8M0 block scales of v_mfma_scale_f32_32x32x64_f8f6f4 undo the 2^-9 on
//    both sides, so one MFMA forms one 64-wide group's integer partial P_g
//    exactly in fp32 (no int->float conversion);
//  - the two-sided scale S = sx (x) sw of a 32x32 block is an outer product;
//    a v_mfma_f32_32x32x16_f16 with a single non-zero k forms it exactly
//    (fp16 x fp16 fits fp32), so the matrix pipe, not the VALU, builds it and
//    the VALU does one FMA per output element per group: acc += P_g * S_g;
//  - packed nibbles are expanded to FP8 once per workgroup while a group is
//    staged into LDS, in MFMA lane order, so each wave reads a 32x64 operand
//    fragment as contiguous 1 KB runs; raw packed data is prefetched three
//    groups ahead in registers;
//  - the tile shape is a template parameter; tiles are swizzled so each XCD
//    (own L2) works on compact groups of tiles;
//  - the accumulator starts from X_hat L1 L2 (bf16 MFMA on the hi/lo split of
//    the fp32 xl1); bias and GELU run in fp32 before the single rounding of
//    the output, which leaves through LDS as row-contiguous 16-byte stores.
#include "common.h"

namespace {

constexpr int FRAG_DW = 8;                   // a 32x64 fp8 fragment: 8 dwords per lane

template <int BM_, int BN_, int WGM_, int WGN_, int MINB_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, MINB = MINB_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int TM = BM / 32 / WGM, TN = BN / 32 / WGN;     // 32x32 blocks per wave
    static constexpr int ABLK = BM / 32, BBLK = BN / 32;
    static constexpr int NA = (ABLK + NW - 1) / NW, NB = (BBLK + NW - 1) / NW;  // blocks staged per wave
    static constexpr int A_DW = ABLK * 64 * FRAG_DW, B_DW = BBLK * 64 * FRAG_DW;
    static constexpr int STAGE_BYTES = 4 * (A_DW + B_DW) + 2 * 64 * (ABLK + BBLK);  // scales [blk][64]
    static constexpr int OUT_LD = BN + 8;
    static constexpr int OUT_BYTES = BM * OUT_LD * 2;
    static constexpr int SMEM_BYTES = (2 * STAGE_BYTES > OUT_BYTES) ? 2 * STAGE_BYTES : OUT_BYTES;
    static_assert(TM * 32 * WGM == BM && TN * 32 * WGN == BN, "tile shape");
};

// the QKV-sized configuration: 256 x 192 tiles, 8 waves (4 x 2) of 64 x 96,
// one workgroup per CU; 4096 x 9216 is 768 tiles = 3 per CU. (Two 4-wave
// workgroups of 128 x 192 per CU measured 1.5x slower: the smaller tile
// stages more bytes per MAC and needs two B staging slots per wave.)
using MainCfg = Cfg<256, 192, 4, 2, 1>;

DEV int out_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <class C>
struct Raw {
    uint4 a[C::NA], b[C::NB];
    uint32_t sa[C::NA], sb[C::NB];
};

struct Stage {
    uint32_t* A;
    uint32_t* B;
    uint16_t* SA;
    uint16_t* SB;
};

template <class C>
DEV Stage stage_ptr(char* smem, int s) {
    char* base = smem + s * C::STAGE_BYTES;
    Stage st;
    st.A = (uint32_t*)base;
    st.B = st.A + C::A_DW;
    st.SA = (uint16_t*)(st.B + C::B_DW);
    st.SB = st.SA + 64 * C::ABLK;
    return st;
}

// Per-thread staging sources. Wave w stages the 32-row blocks w, w + NW, ...
// of the A tile and of the B tile; lane l takes row l % 32 of a block and half
// l / 32 of that row's 32 packed bytes, which is exactly the lane that
// consumes those codes in the MFMA, so fragments are written and read as
// contiguous 1 KB runs (no LDS bank conflicts). Rows past the end are clamped
// to the last row: what they load only reaches output rows or columns that
// are never stored.
template <class C>
struct Src {
    const uint8_t* a[C::NA];
    const uint8_t* b[C::NB];
    const uint16_t* sa[C::NA];
    const uint16_t* sb[C::NB];
};

template <class C, bool SCALES>
DEV void load_raw(Raw<C>& r, const Src<C>& src, int g) {
#pragma unroll
    for (int t = 0; t < C::NA; ++t) {
        r.a[t] = *(const uint4*)(src.a[t] + (int64_t)g * 32);
        r.sa[t] = SCALES ? src.sa[t][g] : 0u;
    }
#pragma unroll
    for (int t = 0; t < C::NB; ++t) {
        r.b[t] = *(const uint4*)(src.b[t] + (int64_t)g * 32);
        r.sb[t] = SCALES ? src.sb[t][g] : 0u;
    }
}

// Fragment layout in LDS: [block][half j][lane][16 bytes]; lane l of block b
// holds the 32 fp8 codes of row 32b + l % 32, k half l / 32.
DEV void expand_store(const uint4& raw, uint32_t* __restrict__ tile, int blk, int lane) {
    uint32_t o[8];
    int4sm_to_fp8(raw.x, o[0], o[1]);
    int4sm_to_fp8(raw.y, o[2], o[3]);
    int4sm_to_fp8(raw.z, o[4], o[5]);
    int4sm_to_fp8(raw.w, o[6], o[7]);
    *(uint4*)(tile + ((blk * 2 + 0) * 64 + lane) * 4) = make_uint4(o[0], o[1], o[2], o[3]);
    *(uint4*)(tile + ((blk * 2 + 1) * 64 + lane) * 4) = make_uint4(o[4], o[5], o[6], o[7]);
}

template <class C>
DEV void store_raw(const Raw<C>& r, const Stage& st, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < C::NA; ++t) {
        const int blk = wave + t * C::NW;
        if (C::NA * C::NW == C::ABLK || blk < C::ABLK) {
            expand_store(r.a[t], st.A, blk, lane);
            if (lane < 32) st.SA[blk * 64 + lane] = (uint16_t)r.sa[t];
        }
    }
#pragma unroll
    for (int t = 0; t < C::NB; ++t) {
        const int blk = wave + t * C::NW;
        if (C::NB * C::NW == C::BBLK || blk < C::BBLK) {
            expand_store(r.b[t], st.B, blk, lane);
            if (lane < 32) st.SB[blk * 64 + lane] = (uint16_t)r.sb[t];
        }
    }
}

DEV v8i read_frag(const uint32_t* __restrict__ tile, int blk, int lane) {
    const uint4 a = *(const uint4*)(tile + ((blk * 2 + 0) * 64 + lane) * 4);
    const uint4 b = *(const uint4*)(tile + ((blk * 2 + 1) * 64 + lane) * 4);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Operand of the outer-product MFMA: only k = 0 (element 0 of lanes 0..31) is
// non-zero (lanes 32..63 read the zero half of the scale row); A and B share
// the k layout, so the product is s_row * s_col. The zero registers of the
// tuple stay in place across groups.
DEV v8h scale_operand(v4i& t, const uint16_t* __restrict__ srow, int lane) {
    t[0] = (int)srow[lane];
    return __builtin_bit_cast(v8h, t);
}

template <class C, int MODE, int ACT>   // MODE 0: bf16 out, 1: fp32 out, 2: integer partials dump
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    const float* __restrict__ xl1, const uint16_t* __restrict__ l2t, int rank,
    const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int64_t M, int64_t N, int64_t K,
    int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* __restrict__ part)
{
    constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN, NT = C::NT;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WGN, wn = wave % C::WGN;

    // tile index: blocks are dealt round-robin to the 8 XCDs; consecutive
    // blocks of one XCD take a compact group of tiles (4 tile rows wide) so
    // the XCD's L2 serves both their activation and weight blocks
    const int64_t mext = (MODE == 2) ? pmc : M, next = (MODE == 2) ? pnc : N;
    const int tiles_n = (int)((next + BN - 1) / BN);
    const int tiles_m = (int)((mext + BM - 1) / BM);
    const int tiles = tiles_n * tiles_m;
    int t = blockIdx.x;
    if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
    int tm, tn;
    {
        constexpr int GM = 4;
        const int grp = t / (GM * tiles_n), first = grp * GM;
        const int gsz = (tiles_m - first) < GM ? (tiles_m - first) : GM;
        tm = first + (t % (GM * tiles_n)) % gsz;
        tn = (t % (GM * tiles_n)) / gsz;
    }
    const int64_t m0 = (MODE == 2 ? pm0 : 0) + (int64_t)tm * BM;
    const int64_t n0 = (MODE == 2 ? pn0 : 0) + (int64_t)tn * BN;
    const int64_t mlim = (MODE == 2) ? pm0 + pmc : M;
    const int64_t nlim = (MODE == 2) ? pn0 + pnc : N;
    const int G = (int)(K / 64);

    Src<C> src;
    {
        const int half = lane >> 5;
#pragma unroll
        for (int u = 0; u < C::NA; ++u) {
            const int blk = (wave + u * C::NW) % C::ABLK;
            const int64_t r = m0 + blk * 32 + (lane & 31);
            const int64_t ra = r < mlim ? r : mlim - 1;
            src.a[u] = qx + ra * (K / 2) + 16 * half;
            src.sa[u] = (MODE != 2) ? sx + ra * G : nullptr;
        }
#pragma unroll
        for (int u = 0; u < C::NB; ++u) {
            const int blk = (wave + u * C::NW) % C::BBLK;
            const int64_t r = n0 + blk * 32 + (lane & 31);
            const int64_t rb = r < nlim ? r : nlim - 1;
            src.b[u] = qw + rb * (K / 2) + 16 * half;
            src.sb[u] = (MODE != 2) ? sw + rb * G : nullptr;
        }
    }

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    constexpr bool SC = (MODE != 2);
    Raw<C> r0, r1, r2;
    // group indices past the end are clamped to the last group: the extra
    // loads are harmless and keep the pipeline free of branches
    load_raw<C, SC>(r0, src, 0);
    load_raw<C, SC>(r1, src, G > 1 ? 1 : G - 1);
    load_raw<C, SC>(r2, src, G > 2 ? 2 : G - 1);

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

    // zero upper halves of the per-block scale rows of both stages (staging
    // never writes them; lanes 32..63 of the scale operands read them)
    constexpr int SBLK = C::ABLK + C::BBLK;
    for (int e = tid; e < 2 * SBLK * 32; e += NT) {
        const int stg = e / (SBLK * 32), blk = (e / 32) % SBLK, l = e % 32;
        const Stage zs = stage_ptr<C>(smem, stg);
        if (blk < C::ABLK) zs.SA[blk * 64 + 32 + l] = 0;
        else zs.SB[(blk - C::ABLK) * 64 + 32 + l] = 0;
    }
    store_raw<C>(r0, stage_ptr<C>(smem, 0), wave, lane);
    __syncthreads();
    v4i so_t[TM], wo_t[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) so_t[i] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < TN; ++j) wo_t[j] = v4i{0, 0, 0, 0};

    const v16f zero = {};
    // One group: stage g+1 from its registers, refill them with group g+3,
    // then run the MFMAs of group g from LDS stage g%2.
    auto step = [&](int g, Raw<C>& rn, Raw<C>& rfill) {
        store_raw<C>(rn, stage_ptr<C>(smem, (g + 1) & 1), wave, lane);
        load_raw<C, SC>(rfill, src, (g + 3 < G) ? g + 3 : G - 1);
        const Stage st = stage_ptr<C>(smem, g & 1);
        v8i a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = read_frag(st.A, wm * TM + i, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = read_frag(st.B, wn * TN + j, lane);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const v8h so = scale_operand(so_t[i], st.SA + (wm * TM + i) * 64, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
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
                    const v8h wo = scale_operand(wo_t[j], st.SB + (wn * TN + j) * 64, lane);
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
                    out[lr * C::OUT_LD + lc] = f32_to_bf16_bits(v);
                }
        }
        __syncthreads();
        constexpr int CHUNKS = BN / 8;              // 16-byte chunks per tile row
        for (int c = tid; c < BM * CHUNKS; c += NT) {
            const int lr = c / CHUNKS, lc = (c % CHUNKS) * 8;
            const int64_t row = m0 + lr, col = n0 + lc;
            if (row < M && col < N)
                *(uint4*)((uint16_t*)y + row * ldy + col) = *(const uint4*)(out + lr * C::OUT_LD + lc);
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

template <class C, int MODE, int ACT>
void launch_mode(hipStream_t stream, const uint8_t* qx, const uint16_t* sx,
                 const uint8_t* qw, const uint16_t* sw, const float* xl1, const uint16_t* l2t,
                 int rank, const uint16_t* bias, void* y, int64_t ldy, int64_t M, int64_t N,
                 int64_t K, int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* p) {
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)gemm_w4a4_kernel<C, MODE, ACT>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM_BYTES);
        attr = true;
    }
    const int64_t mext = (MODE == 2) ? pmc : M, next = (MODE == 2) ? pnc : N;
    const int64_t tiles = ((next + C::BN - 1) / C::BN) * ((mext + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((gemm_w4a4_kernel<C, MODE, ACT>), dim3((unsigned)tiles), dim3(C::NT),
                       C::SMEM_BYTES, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K,
                       pm0, pmc, pn0, pnc, p);
}

}  // namespace

hipError_t launch_gemm_w4a4(const uint8_t* qx, const uint16_t* sx, const uint8_t* qw,
                            const uint16_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                            const uint16_t* bias, int act, void* y, int y_f32, int64_t ldy,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    using C = MainCfg;
    if (y_f32) {
        if (act) launch_mode<C, 1, 1>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
        else launch_mode<C, 1, 0>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
    } else {
        if (act) launch_mode<C, 0, 1>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
        else launch_mode<C, 0, 0>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4_partials(const uint8_t* qx, const uint8_t* qw, int64_t M, int64_t N,
                                     int64_t K, int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                     int32_t* p, hipStream_t stream)
{
    launch_mode<MainCfg, 2, 0>(stream, qx, nullptr, qw, nullptr, nullptr, nullptr, 0, nullptr,
                               nullptr, 0, M, N, K, m0, mc, n0, nc, p);
    return hipGetLastError();
}
