// svdq_gemm_w4a4 kernel: 4-bit x 4-bit group GEMM with per-group fp16 scales,
// the low-rank up-projection and bias in the epilogue (optional GELU).
//
// The pages attribute to the original engine a fusion of the low-rank
// up-projection with the 4-bit matmul (remio.ai page, section "SVDQuant moves
// hard values out of 4-bit"). The CDNA4 design:
//  - INT4 codes in [-7, 7] are exact FP6 E2M3 subnormals (q / 8); with the
//    E8M0 block scale 2^3 on both sides one v_mfma_scale_f32_32x32x64_f8f6f4
//    (FP6 operands run at twice the FP8 rate) forms one 64-wide group's
//    integer partial P_g exactly in fp32;
//  - the stored 4-bit word is the E2M3 operand stream with its zero exponent
//    fields folded out, so a wave turns 16 codes into FP6 with four bit
//    operations right before its MFMAs;
//  - packed rows travel from global memory straight into LDS (buffer loads
//    with an LDS destination), two groups = 64 contiguous bytes per row at a
//    time, into a ring of three pair slots filled two steps ahead, with no
//    registers held; every lane's 16 bytes land where the lane that consumes
//    them in the MFMA reads them;
//  - the two-sided scale S = sx (x) sw of a 32x32 block is an outer product
//    that a v_mfma_f32_32x32x8_f16 with one non-zero k forms exactly; the
//    scales arrive in LDS as the zero-extended first register of that
//    operand (lanes 32..63 read zero), and the VALU does one FMA per output
//    element and group, acc += P_g * S_g;
//  - products and scale products of consecutive blocks alternate between two
//    register sets, so a block's FMAs run while the next block's MFMAs do;
//  - tiles are swizzled so each XCD (own L2) works on compact groups of tiles;
//  - the accumulator starts from X_hat L1 L2 (bf16 MFMA on the hi/lo split of
//    the fp32 xl1); bias and GELU run in fp32 before the single rounding of
//    the output, which leaves through LDS as row-contiguous 16-byte stores.
#include "common.h"

namespace {

template <int BM_, int BN_, int WGM_, int WGN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int TM = BM / 32 / WGM, TN = BN / 32 / WGN;     // 32x32 blocks per wave
    static constexpr int ABLK = BM / 32, BBLK = BN / 32, SBLK = ABLK + NW;
    // One pair slot (two groups): codes [group][block][lane][16 B], then
    // scale operands [group][block][lane][4 B]; blocks are the ABLK A blocks,
    // then one B slot per wave (waves w >= BBLK fill theirs with a copy that
    // nobody reads, so every wave issues the same loads).
    static constexpr int CODES = 2 * SBLK * 1024, SLOT = CODES + 2 * SBLK * 256;
    // bf16 output staging for the epilogue: OUT_ROWS rows at a time in slot 0
    static constexpr int OUT_LD = BN + 8, OUT_ROWS = 32 * TM;
    static_assert(TM * 32 * WGM == BM && TN * 32 * WGN == BN, "tile shape");
    static_assert(ABLK <= NW && BBLK <= NW, "one loaded block per wave and operand");
    static_assert((TM * TN) % 2 == 0, "blocks per wave must be even for the register rotation");
    static_assert(OUT_ROWS * OUT_LD * 2 <= SLOT, "epilogue staging fits one slot");
    static_assert(3 * SLOT <= 160 * 1024, "LDS budget");
};

// the QKV-sized configuration: 256 x 192 tiles, 8 waves (4 x 2) of 64 x 96,
// one workgroup per CU; 4096 x 9216 is 768 tiles = 3 per CU.
using MainCfg = Cfg<256, 192, 4, 2>;

DEV int out_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory into LDS at lds + 16 * lane
DEV void dma16(rsrc_t r, char* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// 2 bytes per lane into the low half of the dword at lds + 4 * lane (the
// high half is zeroed; lanes whose offset is out of range get 0)
DEV void dma2(rsrc_t r, char* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 2, voff, soff, 0, 0);
}

// 16 raw bytes (two stored words) -> the lane's FP6 fragment (6 dwords)
DEV v6i unfold_frag(const uint4& raw) {
    uint32_t d[6];
    unfold_fp6(raw.x, raw.y, d[0], d[1], d[2]);
    unfold_fp6(raw.z, raw.w, d[3], d[4], d[5]);
    return v6i{(int)d[0], (int)d[1], (int)d[2], (int)d[3], (int)d[4], (int)d[5]};
}

template <class C, int MODE, int ACT>   // MODE 0: bf16 out, 1: fp32 out, 2: integer partials dump
__global__ __launch_bounds__(C::NT, 1) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    const float* __restrict__ xl1, const uint16_t* __restrict__ l2t, int rank,
    const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int64_t M, int64_t N, int64_t K,
    int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* __restrict__ part)
{
    constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN, NT = C::NT;
    // three pair slots as separate objects: the compiler then tracks each
    // slot's outstanding LDS-destination loads on its own and makes reads of
    // one slot wait only for loads into that slot
    __shared__ __attribute__((aligned(16))) char slot0[C::SLOT];
    __shared__ __attribute__((aligned(16))) char slot1[C::SLOT];
    __shared__ __attribute__((aligned(16))) char slot2[C::SLOT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int G = (int)(K / 64), NP = (G + 1) / 2;   // groups, group pairs

    // Loading: wave w loads block w of the A tile and block w % BBLK of the
    // B tile; lane l takes row l % 32 and half l / 32 of each group of
    // that row, which is where the lane that consumes those codes in the MFMA
    // reads them. Scale loads go to lanes 0..31 (lanes 32..63 get an out-of-
    // range offset, hence 0). Rows past the end are clamped to the last row:
    // what they load only reaches output rows or columns that are never
    // stored. Byte offsets fit in 31 bits (checked on the host).
    const int half = lane >> 5;
    int64_t ra = m0 + (int64_t)(wave % C::ABLK) * 32 + (lane & 31);
    int64_t rb = n0 + (int64_t)(wave % C::BBLK) * 32 + (lane & 31);
    ra = ra < mlim ? ra : mlim - 1;
    rb = rb < nlim ? rb : nlim - 1;
    const rsrc_t rqa = make_rsrc(qx, M * (K / 2));
    const rsrc_t rqb = make_rsrc(qw, N * (K / 2));
    const rsrc_t rsa = make_rsrc(sx, (MODE != 2) ? M * G * 2 : 0);
    const rsrc_t rsb = make_rsrc(sw, (MODE != 2) ? N * G * 2 : 0);
    const int va = (int)(ra * (K / 2)) + 16 * half, vb = (int)(rb * (K / 2)) + 16 * half;
    constexpr int OUT_OF_RANGE = 0x7FFFFFF0;
    const int vsa = half ? OUT_OF_RANGE : (int)(ra * G * 2);
    const int vsb = half ? OUT_OF_RANGE : (int)(rb * G * 2);

    // pair q into a slot (pair indices past the end are clamped; groups past
    // the end get a zero scale operand where they are read).
    auto load_pair = [&](char* sl, int q) {
        q = q < NP ? q : NP - 1;
        const int so = q * 64, ss = q * 4;
        dma16(rqa, sl + (0 * C::SBLK + wave) * 1024, va, so);
        dma16(rqa, sl + (1 * C::SBLK + wave) * 1024, va + 32, so);
        if constexpr (MODE != 2) {
            dma2(rsa, sl + C::CODES + (0 * C::SBLK + wave) * 256, vsa, ss);
            dma2(rsa, sl + C::CODES + (1 * C::SBLK + wave) * 256, vsa + 2, ss);
        }
        dma16(rqb, sl + (0 * C::SBLK + C::ABLK + wave) * 1024, vb, so);
        dma16(rqb, sl + (1 * C::SBLK + C::ABLK + wave) * 1024, vb + 32, so);
        if constexpr (MODE != 2) {
            dma2(rsb, sl + C::CODES + (0 * C::SBLK + C::ABLK + wave) * 256, vsb, ss);
            dma2(rsb, sl + C::CODES + (1 * C::SBLK + C::ABLK + wave) * 256, vsb + 2, ss);
        }
    };
    // Wait until this wave's loads of the pair issued two loads back have
    // landed (one pair's loads may stay in flight), then publish with a
    // barrier. The partials dump also stores in the loop, so it waits for all.
    auto publish = [&]() {
        if constexpr (MODE == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        lds_barrier();
    };

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    load_pair(slot0, 0);
    load_pair(slot1, 1);
    load_pair(slot2, 2);

    // low-rank branch while the first pairs are in flight: acc = xl1 L2
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

    // Operands of the group being computed: FP6 fragments and the scale
    // operands {s, 0} (the zero register stays in place). Right after the
    // last MFMA of a group that reads an operand, its raw codes and scale for
    // the next group are read; the codes are turned into FP6 just before
    // their first MFMA there, so in between only the raw registers are live.
    const int l16 = lane * 16, l4 = lane * 4;
    const int ablk = wm * TM, bblk = C::ABLK + wn * TN;
    v6i fa[TM], fb[TN];
    v2i so[TM], wo[TN];
    uint4 ra_n[TM], rb_n[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) so[i] = v2i{0, 0};
#pragma unroll
    for (int j = 0; j < TN; ++j) wo[j] = v2i{0, 0};
    // operand i / j of group gi (0 / 1) of the pair in slot sl; `phantom`:
    // that group lies past the end of K
    auto read_a = [&](const char* sl, int gi, int i, bool phantom) {
        ra_n[i] = *(const uint4*)(sl + (gi * C::SBLK + ablk + i) * 1024 + l16);
        if constexpr (MODE != 2) {
            const int s = *(const int*)(sl + C::CODES + (gi * C::SBLK + ablk + i) * 256 + l4);
            so[i][0] = phantom ? 0 : s;
        }
    };
    auto read_b = [&](const char* sl, int gi, int j) {
        rb_n[j] = *(const uint4*)(sl + (gi * C::SBLK + bblk + j) * 1024 + l16);
        if constexpr (MODE != 2)
            wo[j][0] = *(const int*)(sl + C::CODES + (gi * C::SBLK + bblk + j) * 256 + l4);
    };

    const v16f zero = {};
    // products and scale products of consecutive blocks, by parity
    v16f P0 = zero, P1 = zero, S0 = zero, S1 = zero;

    // One group g (raw operands read). For block b = (i, j): operands used
    // for the first time are turned into FP6; the two MFMAs of b, then the
    // FMAs of block b - 1 (for b = 0: the last block of the previous group,
    // parity 1); operands used for the last time are read for the next group
    // (group gi of slot nsl; nph = that group is a phantom).
    auto group = [&](int g, const char* nsl, int gi, bool nph) {
#pragma unroll
        for (int bl = 0; bl < TM * TN; ++bl) {
            const int i = bl / TN, j = bl % TN;
            if (j == 0) fa[i] = unfold_frag(ra_n[i]);
            if (i == 0) fb[j] = unfold_frag(rb_n[j]);
            if constexpr (MODE == 2) {
                order_point(fa[i], fb[j]);
                const v16f p = mfma_fp6_32x32x64(fa[i], fb[j], zero);
                const int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * 32 * TM + i * 32 + out_row(e, lane);
                    if (g < G && row < mlim && col < nlim)
                        part[((row - pm0) * pnc + (col - pn0)) * G + g] = (int32_t)p[e];
                }
            } else {
                const int pb = (bl + TM * TN - 1) % (TM * TN), pi = pb / TN, pj = pb % TN;
                v16f& Pn = (bl & 1) ? P1 : P0;
                v16f& Sn = (bl & 1) ? S1 : S0;
                const v16f& Pp = (bl & 1) ? P0 : P1;
                const v16f& Sp = (bl & 1) ? S0 : S1;
                order_point(fa[i], fb[j]);
                Pn = mfma_fp6_32x32x64(fa[i], fb[j], zero);
                order_point(so[i], wo[j]);
                Sn = mfma_f16_32x32x8(__builtin_bit_cast(v4h, so[i]), __builtin_bit_cast(v4h, wo[j]), zero);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[pi][pj][e] = __builtin_fmaf(Pp[e], Sp[e], acc[pi][pj][e]);
                order_point(acc[pi][pj]);
            }
            if (j == TN - 1) read_a(nsl, gi, i, nph);
            if (i == TM - 1) read_b(nsl, gi, j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: pair 0 published (pairs 1 and 2 may stay in flight), group
    // 0's operands read
    if constexpr (MODE == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    lds_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(slot0, 0, i, false);
#pragma unroll
    for (int j = 0; j < TN; ++j) read_b(slot0, 0, j);

    // Step q (pair q in slot q % 3): group 2q, during which group 2q + 1's
    // operands are read; publish pair q + 1 (loaded two steps ago); load
    // pair q + 3 into pair q's slot, which nobody reads any more; group
    // 2q + 1, during which group 2q + 2's operands are read from pair q + 1.
    // The step count is rounded up to a multiple of three so the loop body
    // has no branches (which would blur the compiler's per-slot tracking of
    // loads into LDS); the extra groups carry zero scales.
    auto step = [&](int q, char* cur, char* nxt) {
        group(2 * q, cur, 1, 2 * q + 1 >= G);
        publish();
        load_pair(cur, q + 3);
        group(2 * q + 1, nxt, 0, 2 * q + 2 >= G);
    };
    for (int q = 0; q < NP; q += 3) {
        step(q, slot0, slot1);
        step(q + 1, slot1, slot2);
        step(q + 2, slot2, slot0);
    }
    if constexpr (MODE != 2) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[TM - 1][TN - 1][e] = __builtin_fmaf(P1[e], S1[e], acc[TM - 1][TN - 1][e]);
    }
    // every load into LDS has landed and every wave is done with the slots
    __syncthreads();

    if constexpr (MODE == 0) {
        // bias, GELU and bf16 rounding in registers, then transposed through
        // LDS (slot 0), one wave row (OUT_ROWS rows) at a time, for
        // row-contiguous stores
        uint32_t ob[TM][TN][8];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
            const float bv = (bias && col < N) ? bf16_lo_to_f32(bias[col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    float v0 = acc[i][j][e] + bv, v1 = acc[i][j][e + 1] + bv;
                    if constexpr (ACT == 1) { v0 = gelu_tanh_f32(v0); v1 = gelu_tanh_f32(v1); }
                    ob[i][j][e / 2] = pack_bf16x2(v0, v1);
                }
        }
        uint16_t* out = (uint16_t*)slot0;
        constexpr int CHUNKS = BN / 8;              // 16-byte chunks per tile row
        for (int r = 0; r < C::WGM; ++r) {
            if (wm == r) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int lc = wn * 32 * TN + j * 32 + (lane & 31);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int lr = i * 32 + out_row(e, lane);
                            out[lr * C::OUT_LD + lc] = (uint16_t)(ob[i][j][e / 2] >> (16 * (e & 1)));
                        }
                }
            }
            __syncthreads();
            for (int c = tid; c < C::OUT_ROWS * CHUNKS; c += NT) {
                const int lr = c / CHUNKS, lc = (c % CHUNKS) * 8;
                const int64_t row = m0 + r * C::OUT_ROWS + lr, col = n0 + lc;
                if (row < M && col < N)
                    *(uint4*)((uint16_t*)y + row * ldy + col) = *(const uint4*)(out + lr * C::OUT_LD + lc);
            }
            __syncthreads();
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
    const int64_t mext = (MODE == 2) ? pmc : M, next = (MODE == 2) ? pnc : N;
    const int64_t tiles = ((next + C::BN - 1) / C::BN) * ((mext + C::BM - 1) / C::BM);
    hipLaunchKernelGGL((gemm_w4a4_kernel<C, MODE, ACT>), dim3((unsigned)tiles), dim3(C::NT),
                       0, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K,
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
