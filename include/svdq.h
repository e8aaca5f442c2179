/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 linear layer and the
 * AWQ W4A16 GEMV.
 *
 * The method (remio.ai page "Nunchaku Diffusers support cuts VRAM but hardware
 * still sets the rules", section "SVDQuant moves hard values out of 4-bit";
 * donmalab.com page, core-challenge section): activation outliers are moved
 * into the weights by per-input-channel smoothing, a small 16-bit low-rank
 * branch carries the hardest part of the smoothed weight, the residual runs
 * with 4-bit weights and 4-bit activations, and the two results are added:
 *
 *     X_hat = X diag(inv_lambda)
 *     Y     = X_hat L1 L2  +  sum_g sx[m,g] sw[n,g] P_g[m,n]  +  bias      (-> GELU)
 *     P_g   = sum_{k in group g} qx[m,k] qw[n,k]          (exact integers)
 *
 * Attention and MLP projections take this W4A4 path; adaLN / modulation
 * projections take AWQ W4A16 (4-bit weights, 16-bit activations) -- same
 * pages, sections on the two layer types.
 *
 * Common conventions
 *  - Every pointer is a DEVICE pointer owned by the caller; the library never
 *    allocates, frees or keeps per-call state.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work
 *    and return at once; they never synchronise. Stream order carries the
 *    act -> GEMM dependency.
 *  - Arguments are validated on the host before any HIP call. A failed check
 *    returns its status and launches nothing; svdq_last_error() gives the
 *    detail. There is no fallback path of any kind.
 *  - M == 0 is valid: after the shape checks the call returns SVDQ_OK
 *    without reading any pointer or touching the device.
 *  - Group size is 64 along K; K must be a multiple of 64.
 *  - SVDQ 4-bit codes (format v2): codes in [-7, 7], rows K-contiguous, every
 *    16 consecutive codes of a row form one little-endian 64-bit word (so a
 *    64-wide group is 32 bytes). Put the 16 codes into a 96-bit stream T as
 *    FP6 E2M3 fields (code e at bits 6e..6e+5: |q| in bits 6e..6e+2, zero
 *    exponent bits 6e+3 and 6e+4, sign in bit 6e+5; zero has sign 0). The
 *    word's low dword is T[0:32) | (T[32:64) & 0x18618618) and its high dword
 *    is T[64:96) | (T[32:64) & 0x61861861): the middle third of T rides in the
 *    exponent fields of the outer two, so every bit of the word is a
 *    magnitude or sign bit and any 64-bit pattern is valid. (The layout
 *    follows gfx950's FP6 MFMA operand stream; the pages fix only that codes
 *    are 4-bit.)
 *  - SVDQ group scales (format v3): fp16, "quad-major". With G = K / 64 and
 *    G4 = ceil(G / 4), the scales of a matrix with `rows` rows are an array
 *    [G4][rows][4]: element [q][r][e] is the scale of group 4q + e of row r,
 *    so a row's four scales of one quad are 8 consecutive bytes and the
 *    rows of one quad are contiguous. Groups 4q + e >= G hold 0.
 *  - AWQ 4-bit codes (format v1): unsigned nibbles 0..15, byte i of a row
 *    holds element 2i in bits 0-3 and element 2i+1 in bits 4-7.
 *  - bf16 and fp16 values are passed as their 16-bit patterns.
 *  - Fused projections (the query, key and value projections merged into one
 *    grouped operation, which a loader must map back with a stated tensor
 *    order: remio.ai page, section on the generic integration path): one
 *    layer whose output columns are the projections in order along N
 *    ([Q | K | V]), prepared offline on the concatenated weight (one
 *    smoothing vector, one L1, so one activation pass). Every weight-side
 *    array is indexed by output column and slices along N (qw rows, the
 *    middle axis of the quad-major scales, rows of the [N][r] up-projection,
 *    bias); a slice used with the fused layer's qx, sx and xl1 gives exactly
 *    those output columns.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SVDQ_OK = 0,
    SVDQ_ERR_NULL = 1,        /* a required pointer is NULL                     */
    SVDQ_ERR_SHAPE = 2,       /* size / leading dimension / rank not allowed    */
    SVDQ_ERR_ALIGN = 3,       /* pointer or leading dimension misaligned        */
    SVDQ_ERR_UNSUPPORTED = 4, /* dtype / activation / option not supported      */
    SVDQ_ERR_DEVICE = 5,      /* no device, or the device is not gfx950         */
    SVDQ_ERR_HIP = 6          /* a HIP runtime call or a launch failed          */
} svdq_status;

typedef enum { SVDQ_DT_BF16 = 0, SVDQ_DT_F32 = 1 } svdq_dtype;
typedef enum { SVDQ_ACT_NONE = 0, SVDQ_ACT_GELU_TANH = 1 } svdq_act;

/* Capability check done up front (the remio.ai page, hardware section: the
 * loader verifies GPU capability at start-up and unsupported combinations
 * raise an error instead of running incompatible kernels). Returns SVDQ_OK
 * when `device` exists and is gfx950, else SVDQ_ERR_DEVICE. */
svdq_status svdq_check_device(int device);

/* Static text for a status code; never NULL. */
const char* svdq_status_string(svdq_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* svdq_last_error(void);

/* Library version: format version * 100 + revision. */
int svdq_version(void);

/*
 * svdq_quantize_act -- fused smoothing + rank-r down-projection + INT4
 * group-64 activation quantisation (the remio.ai page, same section: the
 * original engine fused the low-rank down-projection with input quantisation).
 *
 *  x          bf16 [M][ldx], row m's K values contiguous (ldx >= K, ldx % 8 == 0)
 *  inv_lambda fp32 [K] smoothing reciprocals, or NULL for lambda == 1
 *  l1t        the down-projection L1 (K x rank, bf16) in the L1 tile layout
 *             (format v4): an array [K/64][rank/16][2][64][8] whose element
 *             (g, t, s, l, j) is L1[64 g + 16 (l / 16) + 8 s + j][16 t + l % 16],
 *             i.e. for each 64-channel group g, 16-rank tile t and 32-channel
 *             step s, 1 KB in which lane l's 16 bytes are the 8 channels of
 *             rank 16 t + l % 16 that pair with lane l's activation values;
 *             K * rank values in all. NULL iff rank == 0
 *  rank       0..128, multiple of 16
 *  qx         out: packed codes [M][K/2]
 *  sx_f16     out: fp16 scales [ceil(K/256)][M][4] (quad-major, zero padded)
 *  xl1        out: fp32 [M][rank] = X_hat L1 (NULL iff rank == 0)
 *
 * Per element: x_hat = fp32(x) * inv_lambda[k] (one fp32 multiply). Per
 * (row, group): amax = max |x_hat|; s = fp16_rtne(min(amax / 7, 65504));
 * if s == 0 all codes are 0, else q = clamp(rtne(x_hat * fp32(1 / s)), -7, 7).
 * qx and sx are bit-exact with that definition. xl1 is accumulated in fp32
 * (relative error about 1e-6).
 * Alignment: x, inv_lambda, l1t, qx, sx_f16, xl1 16-byte aligned.
 */
svdq_status svdq_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx,
                              const float* inv_lambda, const void* l1t, int32_t rank,
                              uint8_t* qx, void* sx_f16, float* xl1, void* stream);

/*
 * svdq_gemm_w4a4 -- 4-bit x 4-bit group GEMM with the low-rank up-projection,
 * bias and optional GELU(tanh) in the epilogue (the remio.ai page, same
 * section: the up-projection was fused with the 4-bit matmul).
 *
 *  qx, sx_f16  [M][K/2] codes and fp16 [ceil(K/256)][M][4] quad-major scales
 *              from svdq_quantize_act
 *  qw, sw_f16  [N][K/2] weight codes and fp16 [ceil(K/256)][N][4] quad-major
 *              scales (residual R^T); padding groups must hold 0
 *  xl1         fp32 [M][rank] from svdq_quantize_act (NULL iff rank == 0)
 *  l2t         bf16 [N][rank]: row n is column n of L2 (NULL iff rank == 0)
 *  bias        bf16 [N] or NULL
 *  act         SVDQ_ACT_NONE or SVDQ_ACT_GELU_TANH (applied in fp32)
 *  y           out: [M][ldy] of y_dtype (bf16 RTNE of the fp32 result, or fp32)
 *
 * N % 8 == 0, ldy >= N, ldy % 8 == 0; (M + 256) * K / 2, (N + 256) * K / 2,
 * (M + 256) * rank * 4, (N + 256) * rank * 2 and (M + 128) * ldy * (2 or 4
 * bytes) must stay below 2^31 (byte offsets plus a tile of slack). The group partials P_g are exact; the fp32 result
 * matches the fp64 definition to about 1e-6 relative.
 * Alignment: every pointer 16-byte aligned (bias: 2 bytes).
 */
svdq_status svdq_gemm_w4a4(const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                           const uint8_t* qw, const void* sw_f16, int64_t N,
                           const float* xl1, const void* l2t, int32_t rank,
                           const void* bias, int32_t act,
                           void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * MXFP4 form of the same layer (E2M1 codes, one E8M0 exponent per 32 values).
 * The pages run the 4-bit path as INT4 or, on Blackwell, NVFP4 (remio.ai page,
 * loading-path and benchmark sections); this is the microscaled 4-bit float
 * format whose block scales the gfx950 matrix pipe applies itself. The number
 * format follows the OCP Microscaling Formats (MX) Specification v1.0 (E2M1
 * element, E8M0 scale, conversion from FP32); every other step (smoothing,
 * low-rank branch, bias, GELU) is the INT4 layer's.
 *
 * Layouts (format v3, MXFP4 side):
 *  - codes [rows][K/2]: one nibble per value, bit 3 sign, bits 0-2 the E2M1
 *    exponent/mantissa (0, 0.5, 1, 1.5, 2, 3, 4, 6); element 2i in bits 0-3
 *    of byte i, element 2i + 1 in bits 4-7; a zero is stored with sign 0;
 *  - scales: E8M0 bytes (exponent + 127) in [ceil(K/256)][rows][8]: the 8
 *    bytes of (q, r) are the exponents of blocks 8q .. 8q + 7 of row r, even
 *    blocks first (byte 4h + j is block 8q + 2j + h); blocks past K/32 hold 0.
 *
 * svdq_quantize_act_mxfp4: arguments as svdq_quantize_act, with sx_e8m0 the
 * scale array above. Per 32-value block: e = floor(log2(amax)) - 2 clamped to
 * [-127, 127] (-127 for a block of zeros); each value x_hat * 2^-e rounded to
 * the nearest E2M1 value, ties to mantissa 0, saturating at +-6. qx and
 * sx_e8m0 are bit-exact with that definition; xl1 as for INT4.
 */
svdq_status svdq_quantize_act_mxfp4(const void* x, int64_t M, int64_t K, int64_t ldx,
                                    const float* inv_lambda, const void* l1t, int32_t rank,
                                    uint8_t* qx, void* sx_e8m0, float* xl1, void* stream);

/*
 * svdq_gemm_mxfp4: arguments, limits and errors as svdq_gemm_w4a4, with
 * MXFP4 codes and E8M0 scale arrays (above) for both operands:
 *   Y = X_hat L1 L2 + sum_k deq(a)[m,k] deq(w)[n,k] + bias   (-> GELU)
 * The block scales are applied by the matrix pipe and the products of one
 * 64-wide step are summed there in fp32 before joining the accumulator, so
 * the result matches the fp64 definition to fp32 accumulation error.
 */
svdq_status svdq_gemm_mxfp4(const uint8_t* qx, const void* sx_e8m0, int64_t M, int64_t K,
                            const uint8_t* qw, const void* sw_e8m0, int64_t N,
                            const float* xl1, const void* l2t, int32_t rank,
                            const void* bias, int32_t act,
                            void* y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * svdq_gemm_w4a4_partials -- test hook: the same device code path as
 * svdq_gemm_w4a4 (same staging, same MFMA) with the scale epilogue replaced
 * by a dump of the exact integer group partials P_g[m, n] for the rectangle
 * rows [m0, m0 + mcount) x columns [n0, n0 + ncount).
 *  p   out: int32 [mcount][ncount][K/64]
 * Same shape limits as svdq_gemm_w4a4.
 */
svdq_status svdq_gemm_w4a4_partials(const uint8_t* qx, int64_t M, int64_t K,
                                    const uint8_t* qw, int64_t N,
                                    int64_t m0, int64_t mcount, int64_t n0, int64_t ncount,
                                    int32_t* p, void* stream);

/*
 * awq_gemv_w4a16 -- AWQ W4A16 GEMV for the adaLN / modulation projections
 * (donmalab.com page, section on the two schemes; remio.ai page, loading-path
 * section): Y = (X diag(inv_s)) dequant(W) + bias with
 * dequant(W)[k, n] = (q[n, k] - z[n, g]) * s[n, g] computed in registers.
 *
 *  x          bf16 [M][K] (1 <= M <= 16, dense rows)
 *  inv_s      fp32 [K] reciprocal activation-aware channel scales, or NULL
 *  qwt        unsigned 4-bit codes in the GEMV tile layout (format v1 AWQ):
 *             [N/16][K/128][16][64 bytes]. Block (t, j, c) holds bytes
 *             64j .. 64j + 63 of the plain packed row of column n = 16t + c
 *             (the codes of groups 2j and 2j + 1; byte i of a plain row holds
 *             element 2i in bits 0-3 and 2i + 1 in bits 4-7), so the 16
 *             columns of a tile and one group pair form one contiguous 1 KB
 *             block. This is a byte permutation of the plain [N][K/2] layout.
 *  scale_f16  fp16 scales and zero_f16 fp16 zero points (integers 0..15),
 *             both in the GEMV tile layout [N/16][K/64][16]: entry (t, g, c)
 *             belongs to column 16t + c and group g.
 *  bias       bf16 [N] or NULL
 *  y          out: bf16 [M][N]
 * N % 16 == 0, K % 128 == 0; qwt, scale and zero must each stay below 2 GiB.
 * Accumulation is fp32; the result matches the fp64 definition to about 1e-5
 * relative before the bf16 rounding.
 * Alignment: x, inv_s, qwt, y 16-byte aligned; scale/zero 2 bytes.
 */
svdq_status awq_gemv_w4a16(const void* x, int64_t M, int64_t K, const float* inv_s,
                           const uint8_t* qwt, const void* scale_f16, const void* zero_f16,
                           int64_t N, const void* bias, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
