// awq_gemv_w4a16 kernel: 4-bit weights, 16-bit activations, few rows
// (adaLN / modulation projections; donmalab.com page, section on the two
// schemes). Memory-bound: the packed weights are streamed from HBM once and
// dequantised in registers.
//
// CDNA4 design:
//  - Weights arrive in a tile layout, codes [N/16][K/128][16 columns][64 B]
//    and scales / zero points [N/16][K/64][16]: the codes of one group pair
//    of 16 columns are one contiguous 1 KB block and their scales 64 B, so
//    every load instruction of a wave reads whole contiguous runs (16 lanes
//    x 16 B per 256 B run streams at full rate; 16 rows x 32 B per
//    instruction reaches less than half of it).
//  - A nibble q becomes the bf16 value 128 + q exactly by OR-ing it into the
//    bf16 pattern of 128.0 (0x4300).
//  - One v_mfma_f32_16x16x32_bf16 consumes 32 codes of each of 16 columns:
//    lanes 0-31 hold codes of group A of the pair, lanes 32-63 of group B.
//    The 16 rows of the A operand are used as [lo/hi][group][4 token rows]:
//    rows 0-3 carry bf16(x~) of group A, rows 4-7 of group B, rows 8-15 the
//    bf16 remainders x~ - hi, each zero where its group's codes are absent.
//    So one MFMA chain yields D = sum x~ (128 + q) of both groups, hi and lo
//    parts apart, and every lane of the result is a useful number.
//  - The zero point and the offset fold out through the per-(row, group)
//    sums of x~: Y += s (D_hi - (128 + z) X_hi) + s (D_lo - (128 + z) X_lo),
//    where X_hi, X_lo come from the same A fragments times a matrix of ones
//    on the MFMA, so they are the sums the MFMA itself sees and each lane
//    folds its own rows.
//  - About one workgroup per CU: workgroup i owns TPW consecutive column
//    tiles (TPW = 1, 2, 4, 5 or 8, template; 5 at 4 x 3072 -> 18432 on 256
//    CUs). Its NW waves (12 for up to 4 token rows and 5 tiles: three per
//    SIMD, two group pairs each at K = 3072, every load of a wave in flight
//    at once; 8 otherwise) split the group pairs into NW parts; wave w streams
//    part w of every tile of the workgroup,
//    pair-major with the tile index a
//    compile-time constant, so each tile keeps its own accumulator in
//    registers and the task stream has no branch. Each wave prepares, in its
//    own LDS region, exactly what it reads: x~ = x inv_s (bf16 hi/lo in the
//    A-operand order) for its group pairs and the scales and offsets of its
//    groups of every tile; so no workgroup barrier stands between a wave's
//    data landing and its arithmetic. The first loads are issued before the
//    preparation so the weight stream starts at once; codes, scales and zero
//    points are read with the non-temporal policy. Lanes and parts are summed
//    in LDS in a fixed order at the end (deterministic).
//  - Token rows are processed in quads (NQ = 1, 2 or 4, template): every quad
//    has its own A operand and accumulator; weights are loaded once.
#include "common.h"

namespace {

// Waves per workgroup (= K parts) and (pair, tile) tasks per weight batch
// (rounded down to whole pairs), by token quads: one quad (M <= 4) runs 12
// waves of two pairs each at K = 3072 (three waves per SIMD fit its
// registers); more quads, or more than 5 tiles per workgroup, keep more
// accumulators and run 8 waves.
__host__ __device__ constexpr int nw_of(int NQ, int TPW) { return (NQ == 1 && TPW <= 5) ? 12 : 8; }
__host__ __device__ constexpr int btmax_of(int NQ, int TPW) { return nw_of(NQ, TPW) == 12 ? 10 : 16; }
constexpr int ABLK = 528;         // A block per (quad, pair, step): 32 slots x 16 B + zero slot
constexpr int MAXT = 8;           // largest tiles-per-workgroup instantiation
constexpr int LDS_BUDGET = 147456;

__host__ __device__ inline int quads(int M) { return M <= 4 ? 1 : (M <= 8 ? 2 : 4); }

// reduction buffer: [TPW tiles][NW parts][NQ][4 rows][16 columns] floats
__host__ __device__ inline int red_bytes(int NQ, int TPW) { return TPW * nw_of(NQ, TPW) * NQ * 4 * 16 * 4; }

// group pairs held in LDS per chunk: A blocks 4 * ABLK per quad, and
// (scale, offset) pairs 2 groups x 16 TPW columns x 8 B, beside the reduction buffer
__host__ __device__ inline int chunk_pairs(int NQ, int TPW, int KP) {
    const int cp = (LDS_BUDGET - red_bytes(NQ, TPW)) / (4 * ABLK * NQ + 2 * 16 * TPW * 8);
    return KP < cp ? KP : cp;
}

// MFMA slot j of a step holds element perm(j) of the lane's 8 codes, because
// the 8 nibbles of a dword are expanded as pairs (t, t + 4).
DEV int slot_of(int o) { return (o < 4) ? 2 * o : 2 * (o - 4) + 1; }

DEV uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | c; }

// Two dwords of codes at once: one 64-bit shift serves both dwords (the bits
// that cross from the high dword into the low one fall outside the nibble
// mask), so 16 codes take 3 shifts instead of 6.
DEV void codes2_to_bf16(uint32_t x0, uint32_t x1, uint32_t magic, v8bf& b0, v8bf& b1) {
    const uint64_t v = ((uint64_t)x1 << 32) | x0;
    uint64_t s4, s8, s12;
    asm("v_lshrrev_b64 %0, 4, %1" : "=v"(s4) : "v"(v));
    asm("v_lshrrev_b64 %0, 8, %1" : "=v"(s8) : "v"(v));
    asm("v_lshrrev_b64 %0, 12, %1" : "=v"(s12) : "v"(v));
    b0 = __builtin_bit_cast(v8bf, make_uint4(and_or(x0, 0x000F000Fu, magic), and_or((uint32_t)s4, 0x000F000Fu, magic),
                                             and_or((uint32_t)s8, 0x000F000Fu, magic),
                                             and_or((uint32_t)s12, 0x000F000Fu, magic)));
    b1 = __builtin_bit_cast(v8bf, make_uint4(and_or(x1, 0x000F000Fu, magic), and_or((uint32_t)(s4 >> 32), 0x000F000Fu, magic),
                                             and_or((uint32_t)(s8 >> 32), 0x000F000Fu, magic),
                                             and_or((uint32_t)(s12 >> 32), 0x000F000Fu, magic)));
}

DEV uint4 ld128(rsrc_t r, int off, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// read-once data (codes, scales, zero points): non-temporal, so the stream
// does not push x and inv_s (read by every workgroup) out of L2
DEV uint4 ld128_stream(rsrc_t r, int off, int soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 2);   // nt
    return make_uint4(v[0], v[1], v[2], v[3]);
}

DEV uint32_t pk(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

template <int NQ, int TPW>
__global__ __launch_bounds__(64 * nw_of(NQ, TPW), nw_of(NQ, TPW) == 12 ? 1 : 2) void gemv_w4a16_kernel(
    const uint16_t* __restrict__ x, int M, int K, const float* __restrict__ inv_s,
    const uint8_t* __restrict__ qwt, const uint16_t* __restrict__ scale_t,
    const uint16_t* __restrict__ zero_t, int N, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y)
{
    constexpr int LNQ = NQ == 1 ? 0 : (NQ == 2 ? 1 : 2);
    constexpr int NW = nw_of(NQ, TPW), NT = 64 * NW, BTMAX = btmax_of(NQ, TPW);
    // token rows per x~ preparation item (8 channels each): two with 12 waves
    // (whose two pairs of one row quad are then 64 items, one per lane), else four
    constexpr int RPI = NW == 12 ? 2 : 4, LRH = RPI == 2 ? 1 : 0;
    constexpr int PB = ((BTMAX / NQ) / TPW > 0) ? (BTMAX / NQ) / TPW : 1;   // pairs per batch
    constexpr int BT = PB * TPW;                                           // tasks per batch
    constexpr int TC = TPW * 16;                                           // columns per workgroup
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int KP = K / 128, G = K / 64, T = N / 16;
    const int CP = chunk_pairs(NQ, TPW, KP);
    // LDS: A blocks [NQ][CP][4 steps][ABLK], (scale, 128 + zero) [2 CP][TC], reduction buffer
    char* s_a = smem;
    float2* s_so = (float2*)(smem + NQ * CP * 4 * ABLK);
    float* s_red = (float*)(smem + LDS_BUDGET - red_bytes(NQ, TPW));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int c = lane & 15, p = lane >> 4;
    const int t0 = blockIdx.x * TPW;                            // this workgroup's tiles t0 .. t0 + TPW - 1

    // buffer resources (the host checks every array fits 31-bit byte offsets)
    const rsrc_t rw = make_rsrc(qwt, (int64_t)N * (K / 2));
    const rsrc_t rx = make_rsrc(x, (int64_t)M * K * 2);
    const rsrc_t rs = make_rsrc(inv_s, inv_s ? (int64_t)K * 4 : 0);
    const rsrc_t rsc = make_rsrc(scale_t, (int64_t)N * G * 2);
    const rsrc_t rzr = make_rsrc(zero_t, (int64_t)N * G * 2);

    // opaque copy of the bf16 pattern of 128.0 in a VGPR, so the nibble
    // expansion is one v_and_or_b32 per dword (mask from an SGPR)
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic));
    const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

    // A operand: lane (row r, k-group p) reads slot p * 8 + (r >> 3) * 4 + (r & 3)
    // when row r's group (bit 2 of r) matches the lane's codes (p >> 1), else the zero slot
    const int aoff = (((c >> 2) & 1) == (p >> 1)) ? 16 * (p * 8 + (c >> 3) * 4 + (c & 3)) : 512;
    // epilogue: lane (column c, p) holds result rows 4p..4p+3 = [lo/hi][group][row]
    const int eg = p & 1;                      // group of the pair this lane's result belongs to
    const int woff = c * 64 + 16 * p;          // + (tile * KP + pair) * 1024

    v4f acc[TPW][NQ];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[t][q] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int pc0 = 0; pc0 < KP; pc0 += CP) {
        // A wave's preparation (its loads, x~ and the scales into LDS) runs at
        // a raised issue priority, so waves still preparing are not held back
        // by waves already streaming tasks on the same SIMD; it drops back
        // before the task stream (measured: 2.5 % per launch).
        __builtin_amdgcn_s_setprio(3);
        const int np = (KP - pc0) < CP ? (KP - pc0) : CP;       // pairs in this chunk
        const int g0 = 2 * pc0;                                 // first group of this chunk
        // this wave's pairs [ps, pe) of the chunk = its groups [gs, gs + ng); the
        // wave prepares exactly the A blocks and scales it reads itself (no
        // workgroup barrier: each wave starts once its own data has landed)
        const int ps = (wave * np) / NW, pe = ((wave + 1) * np) / NW;
        const int plast = pe > ps ? pe - 1 : ps;
        const int gs = 2 * ps, ng = 2 * (pe - ps), ngd = ng > 0 ? ng : 1;
        const int xitems = ng * NQ * 8 * (4 / RPI);             // (group, quad, RPI rows, 8 channels)
        const int sitems = TPW * ng * 2;                        // (tile, group, 8 columns) uint4

        // ---- 1. preparation loads (x, inv_s; scales, zero points), issued first
        auto xload = [&](int it, uint4 (&xr)[RPI], uint4& s0, uint4& s1) {
            const int itc = it < xitems ? it : (xitems > 0 ? xitems - 1 : 0);   // clamped: in bounds
            const int sub = itc & 7, rh = (itc >> 3) & (4 / RPI - 1), q = (itc >> (3 + LRH)) & (NQ - 1);
            const int gl = gs + (itc >> (3 + LRH + LNQ));
            const int k = (g0 + gl) * 64 + sub * 8;
#pragma unroll
            for (int j = 0; j < RPI; ++j) {
                const int rr = rh * RPI + j;
                const int m = 4 * q + rr;
                const int mr = m < M ? m : M - 1;               // padded rows read a real row
                xr[j] = ld128(rx, (mr * K + k) * 2, 0);
            }
            if (inv_s) {
                s0 = ld128(rs, k * 4, 0);
                s1 = ld128(rs, k * 4 + 16, 0);
            } else {
                s0 = make_uint4(0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u);
                s1 = s0;
            }
        };
        // scale / zero item: 8 columns (half a tile row) of group gl of tile ti
        auto sitem = [&](int it, int& ti, int& gl, int& h) {
            const int itc = it < sitems ? it : (sitems > 0 ? sitems - 1 : 0);
            h = itc & 1;
            const int r = itc >> 1;                             // row (tile, group) of the block
            ti = r / ngd;
            gl = gs + r - ti * ngd;
        };
        auto sload = [&](int it, uint4& sb, uint4& zb) {
            int ti, gl, h;
            sitem(it, ti, gl, h);
            const int tt = t0 + ti < T ? t0 + ti : T - 1;
            const int off = ((tt * G + g0 + gl) * 16 + 8 * h) * 2;
            sb = ld128_stream(rsc, off, 0);
            zb = ld128_stream(rzr, off, 0);
        };
        uint4 xr0[RPI], xs0, xs1, sb0, zb0, sb1, zb1;
        xload(lane, xr0, xs0, xs1);
        sload(lane, sb0, zb0);
        sload(lane + 64, sb1, zb1);
        // keep these ahead of the weight loads: loads complete in issue order,
        // so waiting for a preparation load must not wait for the weights
        __builtin_amdgcn_sched_barrier(0);

        // preparation into LDS: x~ = x inv_s as bf16 hi/lo in A-operand
        // order, and (scale, 128 + zero) per (group, column)
        auto xprep = [&](const uint4 (&xr)[RPI], const uint4& s0, const uint4& s1, int it) {
            if (it >= xitems) return;
            const int sub = it & 7, rh = (it >> 3) & (4 / RPI - 1), q = (it >> (3 + LRH)) & (NQ - 1);
            const int gl = gs + (it >> (3 + LRH + LNQ));
            // channels 8 sub .. 8 sub + 7 of group gl: lane p = 2 (gl & 1) + (sub >> 2), step sub & 3
            const int pl = 2 * (gl & 1) + (sub >> 2), st = sub & 3;
            char* blk = s_a + ((q * CP + (gl >> 1)) * 4 + st) * ABLK;
            const uint32_t sr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int j = 0; j < RPI; ++j) {
                const int rr = rh * RPI + j;
                const uint32_t w[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
                uint16_t hi[8], lo[8];
#pragma unroll
                for (int o = 0; o < 8; ++o) {
                    const float xf = (o & 1) ? bf16_hi_to_f32(w[o >> 1]) : bf16_lo_to_f32(w[o >> 1]);
                    const float xt = xf * __uint_as_float(sr[o]);
                    const __bf16 h = (__bf16)xt;
                    const __bf16 l = (__bf16)(xt - (float)h);
                    hi[slot_of(o)] = __builtin_bit_cast(uint16_t, h);
                    lo[slot_of(o)] = __builtin_bit_cast(uint16_t, l);
                }
                *(uint4*)(blk + 16 * (pl * 8 + rr)) =
                    make_uint4(pk(hi[0], hi[1]), pk(hi[2], hi[3]), pk(hi[4], hi[5]), pk(hi[6], hi[7]));
                *(uint4*)(blk + 16 * (pl * 8 + 4 + rr)) =
                    make_uint4(pk(lo[0], lo[1]), pk(lo[2], lo[3]), pk(lo[4], lo[5]), pk(lo[6], lo[7]));
            }
        };
        auto sprep = [&](const uint4& sb, const uint4& zb, int it) {
            if (it >= sitems) return;
            int ti, gl, h;
            sitem(it, ti, gl, h);
            const uint32_t sw[4] = {sb.x, sb.y, sb.z, sb.w}, zw[4] = {zb.x, zb.y, zb.z, zb.w};
            float2* dst = s_so + gl * TC + ti * 16 + 8 * h;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float sv = f16_bits_to_f32((uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
                const float zv = f16_bits_to_f32((uint16_t)(zw[j >> 1] >> (16 * (j & 1))));
                dst[j] = make_float2(sv, 128.0f + zv);
            }
        };
        // larger M * K or more tiles: items beyond the ones loaded ahead,
        // prepared before any weight load is issued (waiting for them then
        // never waits for the weight stream, and no control-flow merge
        // happens while weights are in flight)
        for (int it0 = 64; it0 < xitems; it0 += 64) {
            uint4 xr[RPI], s0, s1;
            xload(it0 + lane, xr, s0, s1);
            xprep(xr, s0, s1, it0 + lane);
        }
        for (int it0 = 128; it0 < sitems; it0 += 64) {
            uint4 sb, zb;
            sload(it0 + lane, sb, zb);
            sprep(sb, zb, it0 + lane);
        }

        // ---- 2. this wave's first batch of codes
        uint4 qv[BT];
        auto load_batch = [&](int j0) {                          // j0: first pair (chunk-local)
#pragma unroll
            for (int i = 0; i < BT; ++i) {
                // task i: pair j0 + i / TPW, tile t0 + i % TPW; pairs past the end and
                // tiles past N re-read valid data (clamped)
                const int pl = (j0 + i / TPW < pe) ? j0 + i / TPW : plast;
                const int pcl = pc0 + (pl < np ? pl : np - 1);
                const int tt = t0 + i % TPW;
                const int tcl = tt < T ? tt : T - 1;
                // wave-uniform offset: keep it in an SGPR (a VGPR offset would turn
                // each buffer load into a waterfall loop)
                const int wb = __builtin_amdgcn_readfirstlane((tcl * KP + pcl) * 1024);
                qv[i] = ld128_stream(rw, woff, wb);
                __builtin_amdgcn_sched_barrier(0);     // issue in task order (= consumption order)
            }
        };
        load_batch(ps);
        __builtin_amdgcn_sched_barrier(0);

        // ---- 3. preparation into LDS (first items): zero slots of this
        // wave's A blocks, then its x~ and scales. Only this wave reads them,
        // and LDS operations of one wave complete in issue order, so a
        // compiler fence and the wave's own LDS counter are the only waits.
        const int nb = NQ * (pe - ps) * 4;
        for (int b = lane; b < nb; b += 64) {
            const int q = b / ((pe - ps) * 4), rest = b - q * (pe - ps) * 4;
            *(uint4*)(s_a + ((q * CP + ps) * 4 + rest) * ABLK + 512) = make_uint4(0u, 0u, 0u, 0u);
        }
        xprep(xr0, xs0, xs1, lane);
        sprep(sb0, zb0, lane);
        sprep(sb1, zb1, lane + 64);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_setprio(0);

        // ---- 4. stream the tasks, pair by pair: the pair's A fragments are
        // read once and serve its TPW tiles; X (the per-row group sums of
        // hi + lo) comes from the same fragments times ones. No branch: pairs
        // past the end get a zero scale and re-use valid data.
        auto compute = [&](int j0) {
#pragma unroll
            for (int jj = 0; jj < PB; ++jj) {
                const bool live = j0 + jj < pe;                  // wave-uniform
                const int pl = live ? j0 + jj : plast;
                const int g = 2 * pl + eg;
                v8bf a[NQ][4];
                v4f xsum[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        a[q][st] = *(const v8bf*)(s_a + ((q * CP + pl) * 4 + st) * ABLK + aoff);
                        d = mfma_bf16_16x16x32(a[q][st], ones, d);
                    }
                    // rows 4p..4p+3 of this lane: the hi (p < 2) or lo (p >= 2) part
                    // of its group's row sums, folded against the same part of D
                    xsum[q] = d;
                }
#pragma unroll
                for (int ti = 0; ti < TPW; ++ti) {
                    const uint4 qw = qv[jj * TPW + ti];
                    const uint32_t qd[4] = {qw.x, qw.y, qw.z, qw.w};
                    v8bf b[4];
#pragma unroll
                    for (int st = 0; st < 4; st += 2) codes2_to_bf16(qd[st], qd[st + 1], magic, b[st], b[st + 1]);
                    const float2 so = s_so[g * TC + ti * 16 + c];
                    const float sc = live ? so.x : 0.0f;
                    const float oe = so.y;
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int st = 0; st < 4; ++st) d = mfma_bf16_16x16x32(a[q][st], b[st], d);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float t = __builtin_fmaf(-oe, xsum[q][e], d[e]);
                            acc[ti][q][e] = __builtin_fmaf(sc, t, acc[ti][q][e]);
                        }
                    }
                }
                // consume pairs in load order (the tiles of one pair interleave freely):
                // the scheduler does not know that later loads arrive later
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // The first batch (issued before the preparation) is consumed by
        // straight-line code; more pairs continue in a loop whose loads are
        // issued and consumed inside one iteration, so no in-flight register
        // meets another in a merge (which would force an early full wait).
        if (pe > ps) {                    // wave-uniform; a wave without pairs has nothing to add
            compute(ps);
            for (int j0 = ps + PB; j0 < pe; j0 += PB) {
                load_batch(j0);
                compute(j0);
            }
        }
        if (pc0 + CP < KP) __syncthreads();   // LDS reuse by the next chunk (the reduction
                                              // buffer below is a region of its own)
    }

    // ---- 5. sum the 4 lanes of every column (hi/lo, both groups), then the
    // NW parts of every (tile, row, column), in a fixed order
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = acc[t][q][e];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (p == 0) s_red[(((t * NW + wave) * NQ + q) * 4 + e) * 16 + c] = v;
            }
    __syncthreads();
    for (int e = tid; e < TPW * NQ * 4 * 16; e += NT) {
        const int cc = e & 15, r4 = (e >> 4) & 3, q = (e >> 6) & (NQ - 1), ti = e >> (6 + LNQ);
        const int m = 4 * q + r4, nn = (t0 + ti) * 16 + cc;
        float v = 0.0f;
        for (int w = 0; w < NW; ++w) v += s_red[(((ti * NW + w) * NQ + q) * 4 + r4) * 16 + cc];
        if (m < M && nn < N) {
            const float bv = bias ? bf16_lo_to_f32(bias[nn]) : 0.0f;
            y[(int64_t)m * N + nn] = f32_to_bf16_bits(v + bv);
        }
    }
}

template <int NQ, int TPW>
void launch(const uint16_t* x, int M, int K, const float* inv_s, const uint8_t* qwt,
            const uint16_t* scale, const uint16_t* zero, int N, const uint16_t* bias, uint16_t* y,
            hipStream_t stream) {
    // set on every launch (a host-side call, no stream work): the attribute
    // belongs to the current device, and a cached flag would miss a second one
    (void)hipFuncSetAttribute((const void*)gemv_w4a16_kernel<NQ, TPW>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BUDGET);
    const int T = N / 16;
    hipLaunchKernelGGL((gemv_w4a16_kernel<NQ, TPW>), dim3((unsigned)((T + TPW - 1) / TPW)), dim3(64 * nw_of(NQ, TPW)),
                       LDS_BUDGET, stream, x, M, K, inv_s, qwt, scale, zero, N, bias, y);
}

template <int NQ>
void launch_tpw(int tpw, const uint16_t* x, int M, int K, const float* inv_s, const uint8_t* qwt,
                const uint16_t* scale, const uint16_t* zero, int N, const uint16_t* bias, uint16_t* y,
                hipStream_t stream) {
    switch (tpw) {
        case 1: launch<NQ, 1>(x, M, K, inv_s, qwt, scale, zero, N, bias, y, stream); break;
        case 2: launch<NQ, 2>(x, M, K, inv_s, qwt, scale, zero, N, bias, y, stream); break;
        case 4: launch<NQ, 4>(x, M, K, inv_s, qwt, scale, zero, N, bias, y, stream); break;
        case 5: launch<NQ, 5>(x, M, K, inv_s, qwt, scale, zero, N, bias, y, stream); break;
        default: launch<NQ, 8>(x, M, K, inv_s, qwt, scale, zero, N, bias, y, stream); break;
    }
}

}  // namespace

size_t gemv_smem_bytes(int, int64_t) { return LDS_BUDGET; }

// tiles per workgroup: the smallest instantiated count that covers the tiles
// with one workgroup per CU (more workgroups than CUs only past 8 tiles each)
int gemv_tiles_per_wg(int64_t N, int cus) {
    const int64_t T = N / 16;
    const int64_t need = (T + cus - 1) / cus;
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 5 ? 5 : MAXT;
}

hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t K, const float* inv_s,
                             const uint8_t* qwt, const uint16_t* scale, const uint16_t* zero,
                             int64_t N, const uint16_t* bias, uint16_t* y, int cus, hipStream_t stream)
{
    const int tpw = gemv_tiles_per_wg(N, cus);
    switch (quads(M)) {
        case 1: launch_tpw<1>(tpw, x, M, (int)K, inv_s, qwt, scale, zero, (int)N, bias, y, stream); break;
        case 2: launch_tpw<2>(tpw, x, M, (int)K, inv_s, qwt, scale, zero, (int)N, bias, y, stream); break;
        default: launch_tpw<4>(tpw, x, M, (int)K, inv_s, qwt, scale, zero, (int)N, bias, y, stream); break;
    }
    return hipGetLastError();
}
