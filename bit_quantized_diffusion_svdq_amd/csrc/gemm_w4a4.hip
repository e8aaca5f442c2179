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
//    with an LDS destination) four groups at a time: one load instruction
//    covers whole 128-byte lines of 8 rows (the vector memory pipeline's cost
//    follows the number of lines an instruction touches), and the chunk a
//    lane fetches is XOR-swizzled so the lanes that consume a group in the
//    MFMA read LDS without bank conflicts; the scales are stored quad-major
//    (the four scales of a row's quad are 8 bytes, the rows of one quad are
//    contiguous), so one 1 KB load brings a quad's scales for 128 rows and
//    one 8-byte LDS read gives a lane all four;
//  - the two-sided scale S = sx (x) sw of a 32x32 block is an outer product
//    that a v_mfma_f32_32x32x8_f16 forms exactly: A holds a row's four
//    scales of the quad in k = 0..3, B the column's scale of group g in
//    k = g mod 4 and zeros elsewhere; the VALU does one FMA per output
//    element and group, acc += P_g * S_g;
//  - products and scale products of consecutive blocks alternate between two
//    register sets, so one wave's FMAs for a block run while the matrix pipe
//    works on its next block;
//  - persistent workgroups (two per CU) walk their tiles so each XCD (own L2)
//    works on a compact region; a tile's first loads fly while the previous
//    tile's outputs are stored;
//  - the accumulator starts from X_hat L1 L2 (bf16 MFMA on the hi/lo split of
//    the fp32 xl1); bias and GELU run in fp32 before the single rounding of
//    the output, which is stored straight from the MFMA layout.
#include "common.h"
#include "int4_fields.h"

namespace {

template <int BM_, int BN_, int WGM_, int WGN_, int MINB_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, MINB = MINB_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int TM = BM / 32 / WGM, TN = BN / 32 / WGN;     // 32x32 blocks per wave
    static constexpr int ABLK = BM / 32, BBLK = BN / 32, SBLK = ABLK + BBLK;
    // wave w loads the 32-row blocks w, w + NW, ... of A and of B
    static constexpr int APW = ABLK / NW, BPW = BBLK / NW;
    // One quad slot (four groups): codes [block][8-row part][lane][16 B]
    // (A blocks, then B blocks; see the swizzle at the loads) and, in a slot
    // of its own, the scales [tile row][4] fp16 (A rows, then B rows).
    static constexpr int CODE_SLOT = SBLK * 4096, SC_SLOT = (BM + BN) * 8;
    static_assert(TM * 32 * WGM == BM && TN * 32 * WGN == BN, "tile shape");
    static_assert(APW * NW == ABLK && BPW * NW == BBLK && APW >= 1 && BPW >= 1,
                  "blocks split evenly over the waves");
    static_assert((TM * TN) % 2 == 0, "blocks per wave must be even for the register rotation");
    static_assert(BM * 8 == 1024 && BN * 8 == 1024 && NW % 2 == 0,
                  "a quad's scales of the tile rows are one 64-lane load per side");
    static_assert(2 * (CODE_SLOT + SC_SLOT) * MINB <= 160 * 1024, "LDS budget");
};

// 128 x 128 tiles, 4 waves (2 x 2) of 64 x 64, two workgroups per CU. The
// 64 x 64 wave tile leaves room in 256 VGPRs for the accumulators, two sets
// of products and scale products and the operands; with one wave per SIMD
// per workgroup, the two waves that share a SIMD belong to different
// workgroups, never wait for each other at a barrier and so interleave their
// MFMA and VALU work.
using MainCfg = Cfg<128, 128, 2, 2, 2>;

// Tile t -> (tile row, tile column). Workgroup b runs on XCD b % 8 (the
// dispatcher deals workgroups round-robin to the XCDs), and with the grid a
// multiple of 8 every tile of workgroup b has t % 8 == b % 8. When the tile
// grid splits evenly, XCD x owns one of 2 x 4 regions of it and walks it in
// bands of 8 tile rows, column by column, so the tiles in flight on an XCD
// share 8 tile rows of activations and 8 tile columns of weights in its L2.
// Otherwise: bands of 4 tile rows over the whole grid.
DEV void tile_coords(int t, int tiles_m, int tiles_n, int grid, int& tm, int& tn) {
    if (grid % 8 == 0 && (tiles_m * tiles_n) % 8 == 0 && tiles_m % 2 == 0 && tiles_n % 4 == 0) {
        const int x = t & 7, l = t >> 3, RH = tiles_m >> 1, RW = tiles_n >> 2;
        const int band = l / (8 * RW), first = band * 8;
        const int gsz = (RH - first) < 8 ? (RH - first) : 8;
        const int w = l - band * 8 * RW;
        tm = (x & 1) * RH + first + w % gsz;
        tn = (x >> 1) * RW + w / gsz;
    } else {
        constexpr int GM = 4;
        const int grp = t / (GM * tiles_n), first = grp * GM;
        const int gsz = (tiles_m - first) < GM ? (tiles_m - first) : GM;
        tm = first + (t % (GM * tiles_n)) % gsz;
        tn = (t % (GM * tiles_n)) / gsz;
    }
}

DEV int out_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory into LDS at lds + 16 * lane
DEV void dma16(rsrc_t r, char* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// 16 raw bytes (two stored words) -> the lane's FP6 fragment (6 dwords)
DEV v6i unfold_frag(const uint4& raw) {
    uint32_t d[6];
    unfold_fp6(raw.x, raw.y, d[0], d[1], d[2]);
    unfold_fp6(raw.z, raw.w, d[3], d[4], d[5]);
    return v6i{(int)d[0], (int)d[1], (int)d[2], (int)d[3], (int)d[4], (int)d[5]};
}

// The next layer's activation pass, done by MODE 3 on this layer's output
// H = bf16(act(Y)) (which is not stored): smoothing multiplier inv [N],
// its down-projection L1 [N][rank] in the tile layout of the activation
// kernel (format v4) lt, codes qx [M][N/2] and scales sx of H * inv (INT4:
// format v2 codes, format v3 fp16 scales; MXFP4: E2M1 nibbles and the E8M0
// exponent records of the MXFP4 activation kernel), and per 128-column tile
// of H the partial down-projection part [N/128][M][rank] (fp32).
struct NextAct {
    const float* inv;
    const uint16_t* lt;
    int rank;
    uint8_t* qx;
    uint16_t* sx;
    float* part;
};

// MODE 0: bf16 out, 1: fp32 out, 2: integer partials dump (INT4 only),
// 3: the next layer's activation pass on the bf16 output (same FMT).
// FMT 0: INT4 g64 with fp16 scales; 1: MXFP4 (E2M1 codes, E8M0 per 32).
template <class C, int MODE, int ACT, int FMT = 0>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ qx, const uint16_t* __restrict__ sx,
    const uint8_t* __restrict__ qw, const uint16_t* __restrict__ sw,
    const float* __restrict__ xl1, const uint16_t* __restrict__ l2t, int rank,
    const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int64_t M, int64_t N, int64_t K,
    int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* __restrict__ part, NextAct nx)
{
    constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN, NT = C::NT;
    // two quad slots of codes and two of scales, all separate objects: the
    // compiler then tracks each one's outstanding LDS-destination loads on
    // its own and makes reads of a slot wait only for loads into that slot
    __shared__ __attribute__((aligned(16))) char cs0[C::CODE_SLOT];
    __shared__ __attribute__((aligned(16))) char cs1[C::CODE_SLOT];
    __shared__ __attribute__((aligned(16))) char ss0[C::SC_SLOT];
    __shared__ __attribute__((aligned(16))) char ss1[C::SC_SLOT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WGN, wn = wave % C::WGN;

    // The workgroups are persistent: workgroup b takes tiles b, b + grid,
    // ... (tile_coords places them so each XCD works on a compact region).
    const int64_t mext = (MODE == 2) ? pmc : M, next = (MODE == 2) ? pnc : N;
    const int tiles_n = (int)((next + BN - 1) / BN);
    const int tiles_m = (int)((mext + BM - 1) / BM);
    const int tiles = tiles_n * tiles_m;
    int64_t m0 = 0, n0 = 0;                          // origin of the current tile
    const int64_t mlim = (MODE == 2) ? pm0 + pmc : M;
    const int64_t nlim = (MODE == 2) ? pn0 + pnc : N;
    const int G = (int)(K / 64), NQ = (G + 3) / 4;   // groups, quads of groups

    // ---- loads into LDS ------------------------------------------------
    // Codes: a quad of a row is 128 contiguous bytes. Part i (0..3) of a
    // 32-row block is one load: lane l takes row 8 i + l / 8 of the block and
    // its 16-byte chunk c = (l % 8) ^ f(row), f(row) = (row / 2) % 8, so chunk
    // c of block row r lands at byte 128 r + 16 (c ^ f(r)) of the block's 4 KB.
    // Rows past the end of the matrix fall outside the buffer and read 0
    // (their outputs are never stored). Stepping by 8 rows and by quads goes
    // into the scalar offset. Byte offsets fit in 31 bits (checked on the host).
    const rsrc_t rqa = make_rsrc(qx, M * (K / 2));
    const rsrc_t rqb = make_rsrc(qw, N * (K / 2));
    // scales: [G4][rows][4] fp16, quads past the end read 0
    const rsrc_t rsa = make_rsrc(sx, (MODE != 2) ? (int64_t)((G + 3) / 4) * M * 8 : 0);
    const rsrc_t rsb = make_rsrc(sw, (MODE != 2) ? (int64_t)((G + 3) / 4) * N * 8 : 0);
    const int lr8 = lane >> 3;                       // row within an 8-row part
    const int cpe = (lane & 7) ^ (lr8 >> 1);          // chunk for even parts (f = lr8 / 2)
    const int cpo = cpe ^ 4;                          // odd parts (f = 4 + lr8 / 2)
    int vca_e[C::APW], vca_o[C::APW], vcb_e[C::BPW], vcb_o[C::BPW];
    // Scales: quad q of the tile's A rows is the 1 KB at 8 (q M + m0) and of
    // its B rows the 1 KB at 8 (q N + n0): even waves load A's into the first
    // half of the scale slot, odd waves B's into the second half (waves 2 and
    // 3 repeat waves 0 and 1 with identical bytes, which keeps the loop free
    // of branches). Rows past the end of the matrix read the next quad's
    // scales or 0 (their outputs are never stored).
    const bool sb_side = (wave & 1) != 0;
    const rsrc_t rss = sb_side ? rsb : rsa;
    int vss = 0;
    const int sq_stride = (int)((sb_side ? N : M) * 8);
    // Load d (0 .. NDMA - 1) of quad q into a code slot and a scale slot:
    // the 8-row parts of this wave's A blocks, then of its B blocks, then
    // the scales (groups past the end of K read the next row's codes or 0,
    // and zero scales).
    constexpr int NCODE = (C::APW + C::BPW) * 4, NDMA = NCODE + (MODE != 2 ? 1 : 0);
    auto dma_one = [&](char* cs, char* ss, int q, int d) __attribute__((always_inline)) {
        const int so = q * 128;
        if (d < C::APW * 4) {
            const int k = d / 4, i = d % 4;
            dma16(rqa, cs + (wave + k * C::NW) * 4096 + i * 1024, (i & 1) ? vca_o[k] : vca_e[k],
                  so + 8 * i * (int)(K / 2));
        } else if (d < NCODE) {
            const int k = (d - C::APW * 4) / 4, i = d % 4;
            dma16(rqb, cs + (C::ABLK + wave + k * C::NW) * 4096 + i * 1024, (i & 1) ? vcb_o[k] : vcb_e[k],
                  so + 8 * i * (int)(K / 2));
        } else if constexpr (MODE != 2) {
            dma16(rss, ss + (sb_side ? BM * 8 : 0), vss, q * sq_stride);
        }
    };
    auto load_quad = [&](char* cs, char* ss, int q, int dlo, int dhi) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < NDMA; ++d)
            if (d >= dlo && d < dhi) dma_one(cs, ss, q, d);
    };
    // a quad's loads are issued in two halves, spread over the blocks of
    // two consecutive groups, so the waves of a CU never queue all of them
    // at the texture unit at once
    constexpr int DSPLIT = (NDMA + 1) / 2;
    // Wait for this wave's loads (the quad loaded one step ago) and publish
    // them with a barrier.
    auto publish = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    };
    // The first wait of a tile: the previous tile's output stores (NST per
    // wave) were issued after this tile's first loads, and vector memory
    // operations retire in issue order, so waiting until NST remain waits for
    // the loads and lets the stores drain in the background.
    constexpr int NST = 8;
    bool stores_in_flight = false;
    auto publish_first = [&]() __attribute__((always_inline)) {
        if constexpr (MODE == 0) {
            if (stores_in_flight) {
                asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                stores_in_flight = false;
                lds_barrier();
                return;
            }
        }
        publish();
    };

    // ---- low-rank branch: acc += xl1 L2 -------------------------------------
    // Runs after the main loop, 32 ranks at a time, through code slot 0: the
    // chunk's xl1 rows of the tile (128 B each, fp32) at 0 and its l2t rows
    // (64 B each, bf16) at 16 KB, both brought by line-friendly loads into LDS
    // with the chunks of a row XOR-swizzled (16-byte chunk c of tile row r at
    // position c ^ ((r / 2) % 8) for xl1, c ^ ((r / 4) % 4) for l2t) so the
    // MFMA lanes read them without bank conflicts. The first chunk takes the
    // place of the quad past the end of K in the main loop's prefetch, so it
    // has landed when the loop ends. A last chunk of 16 ranks reads 16 more
    // bytes per row that are never used (or 0 past the end of the array).
    const rsrc_t rxl = make_rsrc(xl1, (MODE != 2) ? M * rank * 4 : 0);
    const rsrc_t rl2 = make_rsrc(l2t, (MODE != 2) ? N * rank * 2 : 0);
    int vxl = 0, vl2 = 0;
    auto load_lr = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            dma16(rxl, cs0 + (wave + 4 * k) * 1024, vxl, k * 32 * rank * 4 + r0 * 4);
#pragma unroll
        for (int k = 0; k < 2; ++k)
            dma16(rl2, cs0 + 16384 + (wave + 4 * k) * 1024, vl2, k * 64 * rank * 2 + r0 * 2);
    };

    // Tile t: its origin and this lane's load offsets, then the loads of its
    // quad 0, which the previous tile's output work overlaps.
    auto start_tile = [&](int t) __attribute__((always_inline)) {
        int tm, tn;
        tile_coords(t, tiles_m, tiles_n, (int)gridDim.x, tm, tn);
        m0 = (MODE == 2 ? pm0 : 0) + (int64_t)tm * BM;
        n0 = (MODE == 2 ? pn0 : 0) + (int64_t)tn * BN;
#pragma unroll
        for (int k = 0; k < C::APW; ++k) {
            const int64_t r = m0 + (int64_t)(wave + k * C::NW) * 32 + lr8;
            vca_e[k] = (int)(r * (K / 2)) + 16 * cpe;
            vca_o[k] = (int)(r * (K / 2)) + 16 * cpo;
        }
#pragma unroll
        for (int k = 0; k < C::BPW; ++k) {
            const int64_t r = n0 + (int64_t)(wave + k * C::NW) * 32 + lr8;
            vcb_e[k] = (int)(r * (K / 2)) + 16 * cpe;
            vcb_o[k] = (int)(r * (K / 2)) + 16 * cpo;
        }
        vss = (int)((sb_side ? n0 : m0) * 8) + 16 * lane;
        vxl = (int)((m0 + 8 * wave + lr8) * rank * 4) + 16 * ((wave & 1) ? cpo : cpe);
        vl2 = (int)((n0 + 16 * wave + (lane >> 2)) * rank * 2) + 16 * ((lane & 3) ^ ((lane >> 4) & 3));
        load_quad(cs0, ss0, 0, 0, NDMA);
    };

    v16f acc[TM][TN];
    auto low_rank = [&]() __attribute__((always_inline)) {
        const int h = lane >> 5, r32l = lane & 31;
        for (int r0 = 0; r0 < rank; r0 += 32) {
            if (r0 > 0 || FMT != 0) {
                load_lr(r0);
                publish();
            }
            const int nks = (rank - r0) >= 32 ? 2 : 1;
            for (int ks = 0; ks < nks; ++ks) {
                v8bf ah[TM], al[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int tr = wm * 32 * TM + i * 32 + r32l;
                    const int sw8 = (tr >> 1) & 7, c0 = 4 * ks + 2 * h;
                    const float4 u0 = *(const float4*)(cs0 + tr * 128 + 16 * (c0 ^ sw8));
                    const float4 u1 = *(const float4*)(cs0 + tr * 128 + 16 * ((c0 + 1) ^ sw8));
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
                    const int tc = wn * 32 * TN + j * 32 + r32l;
                    b[j] = *(const v8bf*)(cs0 + 16384 + tc * 64 + 16 * ((2 * ks + h) ^ ((tc >> 2) & 3)));
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        acc[i][j] = mfma_bf16_32x32x16(ah[i], b[j], acc[i][j]);
                        acc[i][j] = mfma_bf16_32x32x16(al[i], b[j], acc[i][j]);
                    }
            }
            lds_barrier();     // slot 0 is read by every wave before it is refilled
        }
    };

    // ---- operands ---------------------------------------------------------
    // Codes of group gq (0..3) of a quad, for this lane (row r = lane % 32 of
    // a block, half h = lane / 32): chunk 2 gq + h of the row. The LDS
    // addresses are kept whole in registers (wave block + lane chunk) so each
    // read is one instruction with the slot and block as its immediate.
    const int r32 = lane & 31, hh = lane >> 5;
    const int ablk = wm * TM, bblk = C::ABLK + wn * TN;
    int xa[4], xb[4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const int xo = 128 * r32 + 16 * ((2 * gq + hh) ^ ((r32 >> 1) & 7));
        xa[gq] = ablk * 4096 + xo;
        xb[gq] = bblk * 4096 + xo;
        order_point(xa[gq], xb[gq]);
    }
    // scales of the quad: A frag i reads tile row (wm TM + i) 32 + r32, B frag
    // j tile row BM + (wn TN + j) 32 + r32, 8 bytes each
    // (MXFP4: the lane's dword of the record, the exponents of its K half)
    int sra = (wm * TM * 32 + r32) * 8 + (FMT == 1 ? 4 * hh : 0);
    int srb = (BM + wn * TN * 32 + r32) * 8 + (FMT == 1 ? 4 * hh : 0);
    order_point(sra, srb);
    // B's scale operand of group gq: the column's scale in k = gq (lanes
    // 0..31, which hold k = 0..3), zero in every other k; lanes 32..63 hold
    // k = 4..7 and are all zero
    const uint32_t msk_lo = hh ? 0u : 0xffffu, msk_hi = hh ? 0u : 0xffff0000u;
    v6i fa[TM], fb[TN];
    v4i fa4[TM], fb4[TN];
    uint4 ra_n[TM], rb_n[TN];
    uint2 sca[2][TM], scb[2][TN];          // a quad's raw scales, by slot parity
    auto read_a = [&](const char* cs, int gq, int i) __attribute__((always_inline)) {
        ra_n[i] = *(const uint4*)(cs + i * 4096 + xa[gq]);
    };
    auto read_b = [&](const char* cs, int gq, int j) __attribute__((always_inline)) {
        rb_n[j] = *(const uint4*)(cs + j * 4096 + xb[gq]);
    };
    auto read_sa = [&](const char* ss, int par, int i) __attribute__((always_inline)) {
        if constexpr (MODE != 2 && FMT == 0) sca[par][i] = *(const uint2*)(ss + i * 256 + sra);
        if constexpr (FMT == 1) sca[par][i].x = *(const uint32_t*)(ss + i * 256 + sra);
    };
    auto read_sb = [&](const char* ss, int par, int j) __attribute__((always_inline)) {
        if constexpr (MODE != 2 && FMT == 0) scb[par][j] = *(const uint2*)(ss + j * 256 + srb);
        if constexpr (FMT == 1) scb[par][j].x = *(const uint32_t*)(ss + j * 256 + srb);
    };
    // B scale operands, one pair per frag and half of the quad: only the
    // non-zero dword is rewritten per group, the other stays 0
    v2i bso[TN][2];
#pragma unroll
    for (int j = 0; j < TN; ++j) bso[j][0] = bso[j][1] = v2i{0, 0};
    auto b_scale = [&](const uint2& w, int gq, int j) __attribute__((always_inline)) {
        const uint32_t m = (gq & 1) ? msk_hi : msk_lo;
        if (gq < 2) bso[j][0][0] = (int)(w.x & m);
        else bso[j][1][1] = (int)(w.y & m);
        return bso[j][gq >> 1];
    };

    const v16f zero = {};
    // products and scale products of consecutive blocks, by parity
    v16f P0 = zero, P1 = zero, S0 = zero, S1 = zero;

    // One group g = 4 q + gq of the quad whose scales have slot parity par
    // (raw code operands read). For block b = (i, j): operands used for the
    // first time are turned into FP6; the two MFMAs of b, then the FMAs of
    // block b - 1 (for b = 0: the last block of the previous group, parity
    // 1); operands used for the last time are read for the next group (group
    // ngq of the quad in ncs; at the end of a quad, also the next quad's
    // scales from nss, into the other parity).
    auto group = [&](int g, int gq, int par, const char* ncs, const char* nss, int ngq,
                     char* dcs, char* dss, int dq, int dlo, int dhi, bool lrl) __attribute__((always_inline)) {
#pragma unroll
        for (int bl = 0; bl < TM * TN; ++bl) {
            const int i = bl / TN, j = bl % TN;
            if constexpr (FMT == 1) {
                // MXFP4: the raw 16 bytes are the operand; the block scales
                // (byte gq of the lane's exponent dword) apply in the MFMA,
                // which accumulates straight into acc
                if (j == 0) fa4[i] = v4i{(int)ra_n[i].x, (int)ra_n[i].y, (int)ra_n[i].z, (int)ra_n[i].w};
                if (i == 0) fb4[j] = v4i{(int)rb_n[j].x, (int)rb_n[j].y, (int)rb_n[j].z, (int)rb_n[j].w};
                order_point(fa4[i], fb4[j]);
                const int sa = (int)sca[par][i].x, sb = (int)scb[par][j].x;
                switch (gq) {
                    case 0: acc[i][j] = mfma_mxfp4_32x32x64<0, 0>(fa4[i], fb4[j], acc[i][j], sa, sb); break;
                    case 1: acc[i][j] = mfma_mxfp4_32x32x64<1, 1>(fa4[i], fb4[j], acc[i][j], sa, sb); break;
                    case 2: acc[i][j] = mfma_mxfp4_32x32x64<2, 2>(fa4[i], fb4[j], acc[i][j], sa, sb); break;
                    default: acc[i][j] = mfma_mxfp4_32x32x64<3, 3>(fa4[i], fb4[j], acc[i][j], sa, sb); break;
                }
            } else {
            if (j == 0) fa[i] = unfold_frag(ra_n[i]);
            if (i == 0) fb[j] = unfold_frag(rb_n[j]);
            }
            if constexpr (FMT == 1) {
            } else if constexpr (MODE == 2) {
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
                const v2i as = v2i{(int)sca[par][i].x, (int)sca[par][i].y};
                const v2i bs = b_scale(scb[par][j], gq, j);
                order_point(fa[i], fb[j]);
                Pn = mfma_fp6_32x32x64(fa[i], fb[j], zero);
                Sn = mfma_f16_32x32x8(__builtin_bit_cast(v4h, as), __builtin_bit_cast(v4h, bs), zero);
                // both MFMAs issue before the FMAs of the previous block,
                // whose inputs are long complete, so one wave keeps the
                // matrix pipe and the VALU busy at the same time
                __builtin_amdgcn_sched_barrier(0);
                // the two-address VOP2 form issues faster than the VOP3 form
                // the compiler picks for an fma whose result overwrites its
                // addend (measured on gfx950)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(acc[pi][pj][e]) : "v"(Pp[e]), "v"(Sp[e]));
            }
            // this block's share of the loads being spread (the last block
            // takes what is left); or the low-rank chunk in place of them
            if (lrl) {
                if (MODE != 2 && bl == 0 && rank > 0) load_lr(0);
            } else if (dhi > dlo) {
                if (bl < TM * TN - 1) load_quad(dcs, dss, dq, dlo + bl, dlo + bl + 1);
                else load_quad(dcs, dss, dq, dlo + bl, dhi);
            }
            if (j == TN - 1) {
                read_a(ncs, ngq, i);
                if (gq == 3) read_sa(nss, par ^ 1, i);
            }
            if (i == TM - 1) {
                read_b(ncs, ngq, j);
                if (gq == 3) read_sb(nss, par ^ 1, j);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };


    // Step q (quad q in slots cur, scale parity par): group 4q, which also
    // issues the second half of quad q + 1's loads (into the other slots);
    // groups 4q + 1 and 4q + 2, each reading the next group's operands;
    // publish quad q + 1; group 4q + 3, reading group 4q + 4's operands and
    // quad q + 1's scales and issuing the first half of quad q + 2's loads
    // into quad q's slots, which nobody reads any more. The step count is
    // rounded up to an even number so the loop body has no branches (which
    // would blur the compiler's per-slot tracking of loads into LDS); the
    // extra groups have zero scales.
    // tail 1 (the second-to-last step): the first low-rank chunk replaces
    // the first half of the quad past the end; tail 2 (the last step): no
    // loads at all.
    auto step = [&](int q, int par, char* cs, char* ss, char* ncs, char* nss, int tail) __attribute__((always_inline)) {
        const int g0 = 4 * q;
        group(g0, 0, par, cs, ss, 1, ncs, nss, q + 1, tail == 2 ? 0 : DSPLIT, tail == 2 ? 0 : NDMA, false);
        group(g0 + 1, 1, par, cs, ss, 2, cs, ss, 0, 0, 0, false);
        group(g0 + 2, 2, par, cs, ss, 3, cs, ss, 0, 0, 0, false);
        publish();
        group(g0 + 3, 3, par, ncs, nss, 0, cs, ss, q + 2, 0, tail ? 0 : DSPLIT, tail == 1);
    };
    // ---- MODE 3: the next layer's activation pass on this tile's output --------
    // H = bf16(act(Y + bias)) of the tile goes row-major into code slot 1
    // (each wave its 64 x 64 block, the 16-byte chunks of row r XOR-swizzled
    // by r % 8). Then lane l owns row l of its wave's block, whose 64 columns
    // are exactly one group of the next layer's K: x = f32(h) * inv, the
    // group maximum, scale and codes are the lane's own (the same steps as
    // the activation kernel), and the 64 codes leave as four stored words.
    // The next layer's down-projection of these 64 columns runs on the bf16
    // MFMA (x split into bf16 hi + lo) as D[j][row] = L1^T[j][k] x[row][k];
    // the B operand wants lanes l and l + 32 to hold the two 8-column halves
    // of one row, so half of each lane's packs trade places with lane l ^ 32.
    // The two waves of a tile row (wn = 0, 1) hold the tile's two 64-column
    // halves: wn = 1 hands its D to wn = 0 through LDS and wn = 0 stores
    // the sum (its half first) as the tile's partial. (Issuing the next
    // tile's first loads before this work measured no faster, and its
    // registers no longer fit.)
    auto next_act = [&](int64_t tm0, int64_t tn0, const float (&bv)[TN]) __attribute__((always_inline)) {
        char* stg = cs1 + wave * 8192;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = acc[i][j][e] + bv[j];
                    if constexpr (ACT == 1) v = gelu_tanh_f32(v);
                    const int lr = i * 32 + out_row(e, lane), lc = j * 32 + (lane & 31);
                    *(uint16_t*)(stg + lr * 128 + (((lc >> 3) ^ (lr & 7)) << 4) + (lc & 7) * 2) = f32_to_bf16_bits(v);
                }
        const int64_t col0 = tn0 + wn * 64;                 // the lane's group of the next layer
        const int64_t row = tm0 + wm * 64 + lane;
        const int g2 = (int)(col0 >> 6);
        float xh[64];
        float amh[2] = {0.0f, 0.0f};                       // maxima of columns 0-31 and 32-63
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint4 hv = *(const uint4*)(stg + lane * 128 + ((c ^ (lane & 7)) << 4));
            const float4 i0 = *(const float4*)(nx.inv + col0 + 8 * c);
            const float4 i1 = *(const float4*)(nx.inv + col0 + 8 * c + 4);
            const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
            const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float h = (k & 1) ? bf16_hi_to_f32(hw[k >> 1]) : bf16_lo_to_f32(hw[k >> 1]);
                xh[8 * c + k] = h * iv[k];
                amh[c >> 2] = fmaxf(amh[c >> 2], fabsf(xh[8 * c + k]));
            }
        }
        // rows past M fall outside the buffer ranges and are dropped
        const rsrc_t rq = make_rsrc(nx.qx, M * (N / 2));
        const int qo = (int)(row * (N / 2) + col0 / 2);
        if constexpr (FMT == 1) {
            // MXFP4: the row's two 32-column blocks, each with its own E8M0
            // exponent (the activation kernel's per-block step); nibble k of
            // the 32 stored bytes is column col0 + k
            uint32_t wd[8];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int e = mx_block_exponent(amh[b]);
                const float sc = mx_inv_scale(e);
                float t[32];
#pragma unroll
                for (int k = 0; k < 32; ++k) t[k] = xh[32 * b + k] * sc;
#pragma unroll
                for (int w8 = 0; w8 < 4; ++w8) wd[4 * b + w8] = e2m1_x8(t + 8 * w8);
                // exponent records [G/4][M][8]: even blocks of the quad in bytes
                // 0-3, odd blocks in bytes 4-7
                if (row < M) ((uint8_t*)nx.sx)[((int64_t)(g2 >> 2) * M + row) * 8 + 4 * b + (g2 & 3)] = (uint8_t)(e + 127);
            }
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]}, rq, qo, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)wd[4], (int)wd[5], (int)wd[6], (int)wd[7]}, rq, qo + 16, 0, 0);
        } else {
            const float amax = fmaxf(amh[0], amh[1]);
            const float s32 = fminf(amax / 7.0f, 65504.0f);
            const _Float16 s16 = (_Float16)s32;
            const float sf = (float)s16;
            const float invs = (sf > 0.0f) ? 1.0f / sf : 0.0f;
            uint2 wd[4];
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) wd[w4] = codes16_fp6(xh + 16 * w4, invs);
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)wd[0].x, (int)wd[0].y, (int)wd[1].x, (int)wd[1].y},
                                                  rq, qo, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)wd[2].x, (int)wd[2].y, (int)wd[3].x, (int)wd[3].y},
                                                  rq, qo + 16, 0, 0);
            // (the scale array's rows past M belong to the next quad: masked)
            if (row < M) nx.sx[((int64_t)(g2 >> 2) * M + row) * 4 + (g2 & 3)] = __builtin_bit_cast(uint16_t, s16);
        }
        const int r2 = nx.rank;
        const rsrc_t rlt = make_rsrc(nx.lt, (int64_t)r2 * N * 2);
        const int lt_half = lane >> 5;
        // wn = 1 hands its D over in its own staging block (it has read its
        // rows of H already: a wave's LDS operations complete in order)
        char* xch = cs1 + (wm * C::WGN + 1) * 8192;
        float* pp = nx.part + ((tn0 / 128) * M) * (int64_t)r2;
        for (int jb = 0; jb < r2; jb += 32) {
            v16f d[2] = {zero, zero};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                // B: x of step st (columns 16 st .. 16 st + 15) as bf16 hi and
                // lo packs of 8 columns; lane l and lane l ^ 32 trade halves
                // so that the 32-row block mb has rows l % 32 + 32 mb with
                // columns 8 (l / 32) + 0..7 of the step
                v8bf bh[2], bl[2];
                {
                    v8bf oh_lo, ol_lo, oh_hi, ol_hi;          // own row, columns + 0..7 / + 8..15
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const __bf16 a0 = (__bf16)xh[16 * st + k], b0 = (__bf16)xh[16 * st + 8 + k];
                        oh_lo[k] = a0;
                        ol_lo[k] = (__bf16)(xh[16 * st + k] - (float)a0);
                        oh_hi[k] = b0;
                        ol_hi[k] = (__bf16)(xh[16 * st + 8 + k] - (float)b0);
                    }
                    const bool lowlane = lane < 32;          // sends its upper half, keeps its lower
                    const uint4 sh = __builtin_bit_cast(uint4, lowlane ? oh_hi : oh_lo);
                    const uint4 sl = __builtin_bit_cast(uint4, lowlane ? ol_hi : ol_lo);
                    uint4 rh, rl;
                    rh.x = __shfl_xor(sh.x, 32); rh.y = __shfl_xor(sh.y, 32); rh.z = __shfl_xor(sh.z, 32); rh.w = __shfl_xor(sh.w, 32);
                    rl.x = __shfl_xor(sl.x, 32); rl.y = __shfl_xor(sl.y, 32); rl.z = __shfl_xor(sl.z, 32); rl.w = __shfl_xor(sl.w, 32);
                    const v8bf gh = __builtin_bit_cast(v8bf, rh), gl = __builtin_bit_cast(v8bf, rl);
                    bh[0] = lowlane ? oh_lo : gh;
                    bl[0] = lowlane ? ol_lo : gl;
                    bh[1] = lowlane ? gh : oh_hi;
                    bl[1] = lowlane ? gl : ol_hi;
                }
                // A: L1[col0 + 16 st + 8 (l / 32) + 0..7][jr], jr = jb + l % 32,
                // one 16-byte chunk of the tile layout (group g2, 16-rank
                // tile jr / 16, step l / 32, tile lane 16 st + jr % 16);
                // ranks past r2 are zero
                const int jr = jb + (lane & 31);
                const int64_t chunk = (((int64_t)g2 * (r2 / 16) + (jr >> 4)) * 2 + lt_half) * 64 + 16 * st + (jr & 15);
                uint4 araw = make_uint4(0u, 0u, 0u, 0u);
                if (jr < r2) araw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rlt, (int)(chunk * 16), 0, 0));
                const v8bf a = __builtin_bit_cast(v8bf, araw);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    d[mb] = mfma_bf16_32x32x16(a, bh[mb], d[mb]);
                    d[mb] = mfma_bf16_32x32x16(a, bl[mb], d[mb]);
                }
            }
            if (wn == 1) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(float4*)(xch + ((mb * 4 + q) * 64 + lane) * 16) =
                            make_float4(d[mb][4 * q], d[mb][4 * q + 1], d[mb][4 * q + 2], d[mb][4 * q + 3]);
            }
            lds_barrier();
            if (wn == 0) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int64_t prow = tm0 + wm * 64 + mb * 32 + (lane & 31);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 o = *(const float4*)(xch + ((mb * 4 + q) * 64 + lane) * 16);
                        const int j = jb + 8 * q + 4 * (lane >> 5);
                        if (prow < M && j < r2)
                            *(float4*)(pp + prow * r2 + j) = make_float4(d[mb][4 * q] + o.x, d[mb][4 * q + 1] + o.y,
                                                                       d[mb][4 * q + 2] + o.z, d[mb][4 * q + 3] + o.w);
                    }
                }
            }
            lds_barrier();       // the hand-over block is free again for the next chunk
        }
    };

    // ---- the tiles of this workgroup ----------------------------------------
    int t = blockIdx.x;
    start_tile(t);
    for (;;) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        S1 = zero;     // the first group's "previous block" adds nothing
        // bias of the lane's columns, fetched now so its latency is hidden
        float bvj[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * 32 * TN + j * 32 + (lane & 31);
            bvj[j] = (MODE != 2 && bias && col < N) ? bf16_lo_to_f32(bias[col]) : 0.0f;
        }
        // quad 0 published, quad 1 in flight, group 0's operands and quad 0's
        // scales read
        publish_first();
        load_quad(cs1, ss1, 1, 0, DSPLIT);
#pragma unroll
        for (int i = 0; i < TM; ++i) { read_a(cs0, 0, i); read_sa(ss0, 0, i); }
#pragma unroll
        for (int j = 0; j < TN; ++j) { read_b(cs0, 0, j); read_sb(ss0, 0, j); }

        if constexpr (FMT == 0) {
            // the last two steps prefetch the first low-rank chunk in place
            // of the quads past the end of K
            const int NQE = (NQ + 1) & ~1;   // steps run in pairs
            for (int q = 0; q < NQE - 2; q += 2) {
                step(q, 0, cs0, ss0, cs1, ss1, 0);
                step(q + 1, 1, cs1, ss1, cs0, ss0, 0);
            }
            step(NQE - 2, 0, cs0, ss0, cs1, ss1, 1);
            step(NQE - 1, 1, cs1, ss1, cs0, ss0, 2);
        } else {
            // (the MXFP4 form keeps one loop body: a peeled copy of the last
            // steps no longer fits its accumulators in the register budget)
            for (int q = 0; q < NQ; q += 2) {
                step(q, 0, cs0, ss0, cs1, ss1, 0);
                step(q + 1, 1, cs1, ss1, cs0, ss0, 0);
            }
        }
        if constexpr (MODE != 2 && FMT == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[TM - 1][TN - 1][e] = __builtin_fmaf(P1[e], S1[e], acc[TM - 1][TN - 1][e]);
        }
        // INT4: the low-rank chunk in slot 0 was published by the last step.
        // Afterwards every load into LDS has landed and every wave is past
        // its last read of both slots.
        if (MODE != 2 && rank > 0) low_rank();
        else publish();
        // ---- outputs -------------------------------------------------------
        // The next tile's quad 0 goes out first (slot 0 is free), then this
        // tile's outputs: bias, GELU and the one rounding run in registers.
        // bf16 outputs leave through LDS: each wave writes its 64 x 64 values
        // row-major into code slot 1 (free: every wave is past its last read)
        // and reads them back as 16-byte row chunks, so a store instruction
        // writes 8 rows x 128 bytes and a wave needs 8 stores, not one per
        // output element. The next tile's first wait does not wait for them
        // (publish_first): every workgroup finishes its tiles at about the
        // same time, and a wait behind the chip-wide burst of output stores
        // would idle the GPU.
        static_assert(TM == 2 && TN == 2 && C::NW == 4 && C::CODE_SLOT >= 32768,
                      "output staging assumes 64 x 64 wave tiles, 4 waves, 32 KB code slots");
        const int64_t em0 = m0, en0 = n0;
        const bool more = t + (int)gridDim.x < tiles;
        // INT4: the next tile's loads go out before the output work. (The
        // MXFP4 form issues them after it: with the output work behind them
        // its accumulators no longer fit the register budget.)
        constexpr bool EARLY_NEXT = (FMT == 0 && MODE == 0);
        if (EARLY_NEXT && more) start_tile(t + (int)gridDim.x);
        if constexpr (MODE == 0) {
            constexpr int RB = 128, CPR = 8;                   // bytes and 16-byte chunks per staged row
            char* stg = cs1 + wave * 8192;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float v = acc[i][j][e] + bvj[j];
                        if constexpr (ACT == 1) v = gelu_tanh_f32(v);
                        const int lr = i * 32 + out_row(e, lane), lc = j * 32 + (lane & 31);
                        *(uint16_t*)(stg + lr * RB + lc * 2) = f32_to_bf16_bits(v);
                    }
            // the wave reads back only what it wrote (its own LDS operations
            // complete in order)
            uint4 ov[NST];
#pragma unroll
            for (int k = 0; k < NST; ++k) {
                const int q = k * 64 + lane;
                ov[k] = *(const uint4*)(stg + (q / CPR) * RB + (q % CPR) * 16);
            }
            if (!EARLY_NEXT && more) start_tile(t + (int)gridDim.x);
            // rows past M fall outside the buffer range and are dropped;
            // chunks past N (a multiple of 8) are masked
            const rsrc_t ry = make_rsrc(y, M * ldy * 2);
#pragma unroll
            for (int k = 0; k < NST; ++k) {
                const int q = k * 64 + lane;
                const int64_t row = em0 + wm * 64 + q / CPR;
                const int64_t col = en0 + wn * 64 + (q % CPR) * 8;
                if (col < N)
                    __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)ov[k].x, (int)ov[k].y, (int)ov[k].z, (int)ov[k].w},
                                                          ry, (int)((row * ldy + col) * 2), 0, 0);
            }
            stores_in_flight = more;
        } else if constexpr (MODE == 1) {
            // fp32 outputs: straight from the MFMA layout, one store per
            // element (two row segments per instruction; the row step is the
            // scalar offset); rows past M are dropped by the buffer range,
            // columns past N masked. The next tile waits for them.
            const rsrc_t ry = make_rsrc(y, M * ldy * 4);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t col = en0 + wn * 32 * TN + j * 32 + (lane & 31);
                if (col < N) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const int64_t row0 = em0 + wm * 32 * TM + i * 32 + 4 * (lane >> 5);
                        const int vo = (int)((row0 * ldy + col) * 4);
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            float v = acc[i][j][e] + bvj[j];
                            if constexpr (ACT == 1) v = gelu_tanh_f32(v);
                            const int so = (8 * (e >> 2) + (e & 3)) * (int)ldy * 4;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, vo, so, 0);
                        }
                    }
                }
            }
            if (more) start_tile(t + (int)gridDim.x);
        } else if constexpr (MODE == 3) {
            next_act(em0, en0, bvj);
            if (more) start_tile(t + (int)gridDim.x);
        } else {
            if (more) start_tile(t + (int)gridDim.x);
        }

        if (!more) break;
        t += (int)gridDim.x;
    }
}

// compute units of the current device (queried once per device)
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <class C, int MODE, int ACT, int FMT = 0>
void launch_mode(hipStream_t stream, const uint8_t* qx, const uint16_t* sx,
                 const uint8_t* qw, const uint16_t* sw, const float* xl1, const uint16_t* l2t,
                 int rank, const uint16_t* bias, void* y, int64_t ldy, int64_t M, int64_t N,
                 int64_t K, int64_t pm0, int64_t pmc, int64_t pn0, int64_t pnc, int32_t* p,
                 NextAct nx = NextAct{nullptr, nullptr, 0, nullptr, nullptr, nullptr}) {
    const int64_t mext = (MODE == 2) ? pmc : M, next = (MODE == 2) ? pnc : N;
    const int64_t tiles = ((next + C::BN - 1) / C::BN) * ((mext + C::BM - 1) / C::BM);
    // persistent workgroups: MINB per CU
    const int64_t slots = (int64_t)C::MINB * device_cu_count();
    const int64_t grid = tiles < slots ? tiles : slots;
    hipLaunchKernelGGL((gemm_w4a4_kernel<C, MODE, ACT, FMT>), dim3((unsigned)grid), dim3(C::NT),
                       0, stream, qx, sx, qw, sw, xl1, l2t, rank, bias, y, ldy, M, N, K,
                       pm0, pmc, pn0, pnc, p, nx);
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

hipError_t launch_gemm_mxfp4(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw,
                             const uint8_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                             const uint16_t* bias, int act, void* y, int y_f32, int64_t ldy,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    using C = MainCfg;
    const uint16_t* sx16 = (const uint16_t*)sx;
    const uint16_t* sw16 = (const uint16_t*)sw;
    if (y_f32) {
        if (act) launch_mode<C, 1, 1, 1>(stream, qx, sx16, qw, sw16, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
        else launch_mode<C, 1, 0, 1>(stream, qx, sx16, qw, sw16, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
    } else {
        if (act) launch_mode<C, 0, 1, 1>(stream, qx, sx16, qw, sw16, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
        else launch_mode<C, 0, 0, 1>(stream, qx, sx16, qw, sw16, xl1, l2t, rank, bias, y, ldy, M, N, K, 0, 0, 0, 0, nullptr);
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

namespace {

// xl1[m][j] = the sum of part[t][m][j] over the 128-column tiles t, in a
// fixed order: the tiles split into four consecutive ranges, each summed in
// tile order by its own thread (8 loads of 16 bytes in flight), and the four
// range sums added first to last. A workgroup covers 64 groups of four
// consecutive elements (M r is a multiple of 16).
__global__ __launch_bounds__(256) void sum_tile_partials_kernel(const float* __restrict__ part, int T, int64_t n4,
                                                                float* __restrict__ xl1) {
    __shared__ float4 red[4][64];
    const int c = threadIdx.x >> 6, gl = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * 64 + gl;
    const int t0 = c * T / 4, t1 = (c + 1) * T / 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (g < n4) {
        const float4* p = (const float4*)part + g;
        int t = t0;
        for (; t + 8 <= t1; t += 8) {
            float4 b[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) b[u] = p[(int64_t)(t + u) * n4];
#pragma unroll
            for (int u = 0; u < 8; ++u) { v.x += b[u].x; v.y += b[u].y; v.z += b[u].z; v.w += b[u].w; }
        }
        for (; t < t1; ++t) {
            const float4 b = p[(int64_t)t * n4];
            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
        }
    }
    red[c][gl] = v;
    __syncthreads();
    if (c == 0 && g < n4) {
        float4 r = red[0][gl];
#pragma unroll
        for (int k = 1; k < 4; ++k) { r.x += red[k][gl].x; r.y += red[k][gl].y; r.z += red[k][gl].z; r.w += red[k][gl].w; }
        ((float4*)xl1)[g] = r;
    }
}

}  // namespace

int64_t gemm_next_partial_bytes(int64_t M, int64_t N, int rank_next) { return (N / 128) * M * rank_next * 4; }

hipError_t launch_gemm_w4a4_next(const uint8_t* qx, const uint16_t* sx, const uint8_t* qw,
                                 const uint16_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                                 const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                                 const float* inv_next, const uint16_t* l1t_next, int rank_next,
                                 uint8_t* qx_next, uint16_t* sx_next, float* xl1_next, float* part,
                                 hipStream_t stream, int fmt)
{
    using C = MainCfg;
    const NextAct nx{inv_next, l1t_next, rank_next, qx_next, sx_next, part};
    if (fmt == 1) {
        if (act) launch_mode<C, 3, 1, 1>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, nullptr, 0, M, N, K, 0, 0, 0, 0, nullptr, nx);
        else launch_mode<C, 3, 0, 1>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, nullptr, 0, M, N, K, 0, 0, 0, 0, nullptr, nx);
    } else {
        if (act) launch_mode<C, 3, 1>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, nullptr, 0, M, N, K, 0, 0, 0, 0, nullptr, nx);
        else launch_mode<C, 3, 0>(stream, qx, sx, qw, sw, xl1, l2t, rank, bias, nullptr, 0, M, N, K, 0, 0, 0, 0, nullptr, nx);
    }
    if (rank_next > 0) {
        const int64_t n4 = M * rank_next / 4;
        hipLaunchKernelGGL(sum_tile_partials_kernel, dim3((unsigned)((n4 + 63) / 64)), dim3(256), 0, stream, part,
                           (int)(N / 128), n4, xl1_next);
    }
    return hipGetLastError();
}
