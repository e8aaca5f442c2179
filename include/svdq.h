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
typedef enum { SVDQ_FMT_INT4 = 0, SVDQ_FMT_MXFP4 = 1 } svdq_fmt;

/*
 * svdq_layer_desc -- the per-module quantisation settings of one SVDQ layer.
 * The remio.ai page (section on how Diffusers support changes the loading
 * path) describes a quantization config that names, per module, the scheme,
 * the precision, the group size and the low-rank correction; its section on
 * what to watch after the Lite release asks for clear errors on malformed
 * configurations. This struct is that record for one layer:
 *
 *  K, N    input and output widths (K % 64 == 0, N % 8 == 0, both >= 1)
 *  rank    low-rank correction rank r (0..128, multiple of 16; 0 = none)
 *  group   quantisation group along K: must be 64 (the only group size built)
 *  fmt     SVDQ_FMT_INT4 (symmetric INT4, fp16 scale per 64) or
 *          SVDQ_FMT_MXFP4 (E2M1, E8M0 exponent per 32)
 *  act     SVDQ_ACT_NONE or SVDQ_ACT_GELU_TANH (the output epilogue)
 *
 * The caller owns the struct; the library reads it during the call only.
 */
typedef struct {
    int64_t K, N;
    int32_t rank;
    int32_t group;
    int32_t fmt;
    int32_t act;
} svdq_layer_desc;

/*
 * Byte sizes of the weight-side arrays of a layer (what a loader must hand
 * to svdq_gemm_w4a4 / svdq_gemm_mxfp4 and svdq_quantize_act*):
 *  qw      packed codes [N][K/2]
 *  sw      scales: INT4 fp16 [ceil(K/256)][N][4]; MXFP4 E8M0 [ceil(K/256)][N][8]
 *  l1t     down-projection in the L1 tile layout, K * rank bf16 (0 if rank 0)
 *  l2t     up-projection [N][rank] bf16 (0 if rank 0)
 *  inv_lambda  smoothing reciprocals fp32 [K]
 *  bias    bf16 [N]
 * and, for an activation batch of M rows, per row:
 *  qx_row  K/2 bytes; sx_row  ceil(K/256) * 8 bytes; xl1_row  rank * 4 bytes.
 */
typedef struct {
    int64_t qw, sw, l1t, l2t, inv_lambda, bias;
    int64_t qx_row, sx_row, xl1_row;
} svdq_layer_sizes;

/* Check a layer description: NULL -> SVDQ_ERR_NULL; K, N, rank out of the
 * rules above -> SVDQ_ERR_SHAPE; group != 64, unknown fmt or act ->
 * SVDQ_ERR_UNSUPPORTED. The detail names the offending field
 * (svdq_last_error). Touches no device. The compute entry points apply the
 * same rules to their own K, N, rank and act arguments. */
svdq_status svdq_validate_desc(const svdq_layer_desc* desc);

/* Validate `desc`, then fill `sizes` (caller-owned) with the array sizes
 * above. Touches no device. */
svdq_status svdq_layer_sizes_of(const svdq_layer_desc* desc, svdq_layer_sizes* sizes);

/* Capability check done up front (the remio.ai page, hardware section: the
 * loader verifies GPU capability at start-up and unsupported combinations
 * raise an error instead of running incompatible kernels). Returns SVDQ_OK
 * when `device` exists and is gfx950, else SVDQ_ERR_DEVICE. */
svdq_status svdq_check_device(int device);

/* Static text for a status code; never NULL. */
const char* svdq_status_string(svdq_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* svdq_last_error(void);

/* Library version: format version * 100 + revision (404: format 4, revision 4,
 * which adds awq_quantize_weight; revision 3 added
 * svdq_quantize_residual_mxfp4, revision 2 svdq_gemm_mxfp4_quant_next; the
 * formats are unchanged). */
int svdq_version(void);

/*
 * svdq_quantize_act -- fused smoothing + rank-r down-projection + INT4
 * group-64 activation quantisation (the remio.ai page, same section: the
 * original engine fused the low-rank down-projection with input quantisation).
 *
 *  x          bf16 [M][ldx], row m's K values contiguous (K <= ldx < 2^26,
 *             ldx % 8 == 0)
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
 * LDS: ranks up to 32 take any K; ranks 48-128 keep K fp32 reciprocals and
 * per-wave partials in LDS, 4 (K + K/8 + 128 rank) bytes of the 160 KB
 * (K <= 21824 at rank 128), SVDQ_ERR_SHAPE beyond.
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

/*
 * Measurement helpers. They take no part in the layer's arithmetic; a
 * benchmark uses them to state the conditions its figures were taken under
 * (the hysygc.com page, section on speed and image comparisons, asks that
 * a latency figure say what it includes and how it was taken).
 *
 * svdq_probe_clock: one lane spins `spins` short no-op groups (1..1e7) and
 *   writes two int64 values to the device buffer `ticks`: shader-clock ticks
 *   and ticks of the constant 100 MHz real-time counter over the same span,
 *   so clock_MHz = 100 * ticks[0] / ticks[1].
 * svdq_probe_read: reads every byte of the device buffer `buf` once (bytes a
 *   positive multiple of 16 below 2^31, `buf` 16-byte aligned) with
 *   `blocks` (1..65536) workgroups of 256 lanes, and stores one XOR word per
 *   workgroup into `sink` [blocks]: the time of a pure read of that size.
 */
svdq_status svdq_probe_clock(int64_t* ticks, int32_t spins, void* stream);
svdq_status svdq_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/* svdq_gemm_w4a4_quant_next -- svdq_gemm_w4a4 whose output is not stored
 * but quantised for the next layer in the same kernel: H = bf16(act(Y))
 * (act as for svdq_gemm_w4a4; the GELU of an MLP's first linear) is the
 * next layer's input, and the epilogue runs that layer's activation pass
 * on it, with results identical to svdq_quantize_act(H, inv_lambda_next,
 * l1t_next, rank_next) up to the summation order of xl1_next. This is the
 * fusion the remio.ai page names for the original engine (section on
 * SVDQuant moving hard values out of 4-bit: the down-projection fused into
 * input quantisation, so the 16-bit branch adds no separate pass), taken
 * one step further: the 16-bit H of an MLP (113 MB at 4608 x 12288) never
 * goes to memory. The donmalab.com page (section on squeezing out more
 * performance) credits removing such overhead with most of the gain.
 *
 *  this layer   qx, sx_f16, M, K, qw, sw_f16, N, xl1, l2t, rank, bias, act:
 *               as svdq_gemm_w4a4; N a multiple of 128 (whole tiles).
 *  next layer   inv_lambda_next fp32 [N] (16-byte aligned; its input
 *               channels are this layer's outputs), l1t_next its L1 in the
 *               tile layout (format v4, K = N), rank_next a multiple of 16
 *               in [0, 64].
 *  outputs      qx_next [M][N/2] (format v2), sx_next [ceil(N/256)][M][4]
 *               fp16 (format v3, the padding groups of a last partial quad
 *               are not written), xl1_next fp32 [M][rank_next] (16-byte
 *               aligned).
 *  workspace    svdq_gemm_w4a4_quant_next_workspace_size() bytes (16-byte
 *               aligned, contents irrelevant): every 128-column tile's
 *               share of xl1_next, summed afterwards in tile order (so the
 *               result is deterministic). Calls sharing it must not overlap.
 */
svdq_status svdq_gemm_w4a4_quant_next_workspace_size(int64_t M, int64_t N, int32_t rank_next, int64_t* bytes);
svdq_status svdq_gemm_w4a4_quant_next(const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                                      const uint8_t* qw, const void* sw_f16, int64_t N,
                                      const float* xl1, const void* l2t, int32_t rank,
                                      const void* bias, int32_t act,
                                      const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                      uint8_t* qx_next, void* sx_next_f16, float* xl1_next,
                                      void* workspace, int64_t workspace_bytes, void* stream);

/* svdq_gemm_mxfp4_quant_next -- the MXFP4 form of svdq_gemm_w4a4_quant_next:
 * svdq_gemm_mxfp4 whose bf16 output H = bf16(act(Y)) is not stored but
 * quantised for the next MXFP4 layer in the same kernel, with results
 * identical to svdq_quantize_act_mxfp4(H, inv_lambda_next, l1t_next,
 * rank_next) up to the summation order of xl1_next. Arguments, shapes,
 * workspace (svdq_gemm_w4a4_quant_next_workspace_size) and errors as for
 * svdq_gemm_w4a4_quant_next, except the formats: qx, sx, qw, sw as for
 * svdq_gemm_mxfp4; qx_next [M][N/2] E2M1 nibbles and sx_next the E8M0
 * exponent records [ceil(N/256)][M][8] of svdq_quantize_act_mxfp4 (the
 * records' bytes for padding blocks of a last partial quad are not
 * written). A block-level MXFP4 MLP then needs no activation pass for its
 * second linear (the 4-bit floating-point path the remio.ai page names the
 * fastest, section on hardware support dividing the fastest and the widest
 * paths; the fusion as above).
 */
svdq_status svdq_gemm_mxfp4_quant_next(const uint8_t* qx, const void* sx, int64_t M, int64_t K,
                                       const uint8_t* qw, const void* sw, int64_t N,
                                       const float* xl1, const void* l2t, int32_t rank,
                                       const void* bias, int32_t act,
                                       const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                       uint8_t* qx_next, void* sx_next, float* xl1_next,
                                       void* workspace, int64_t workspace_bytes, void* stream);

/* svdq_gemm_w4a4_quant_next_noalloc -- svdq_gemm_w4a4_quant_next for callers
 * that cannot allocate device memory: code recorded under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments
 * without the workspace: the tile partials go to a scratch array built into
 * the library (64 MiB per GPU, held until the process ends; the MLP's fc1 at
 * 4608 tokens, N 12288, rank_next 32, takes 56.6 MB). A call whose partials
 * (N / 128) * M * rank_next * 4 bytes exceed it returns SVDQ_ERR_SHAPE and
 * launches nothing. Nothing in the array needs to start at zero (every call
 * writes all it reads). Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race; order
 * them on one stream. Allocates nothing (no hipMalloc, no allocating
 * library routine). */
svdq_status svdq_gemm_w4a4_quant_next_noalloc(const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                                              const uint8_t* qw, const void* sw_f16, int64_t N,
                                              const float* xl1, const void* l2t, int32_t rank,
                                              const void* bias, int32_t act,
                                              const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                              uint8_t* qx_next, void* sx_next_f16, float* xl1_next, void* stream);

/* ------------------------------------------------------------------------
 * Offline quantiser: turning a bf16 weight into the arrays above, on the
 * GPU. This is the Quantize step of the tool chain the donmalab.com page
 * describes (section on quantising a model yourself: inspect, quantize,
 * package, validate), with the roles the remio.ai page gives the parts
 * (section on SVDQuant moving hard values out of 4-bit): calibration
 * statistics set the smoothing, a 16-bit low-rank branch takes the hardest
 * part of the smoothed weight, the residual becomes 4-bit. Every call
 * enqueues on `stream`, allocates nothing and does not synchronise; all
 * pointers are device memory owned by the caller. Results are
 * deterministic (no atomics on floating-point sums).
 *
 * svdq_calib_absmax -- per-channel absolute maxima of a bf16 matrix
 *   a [rows][cols] (row stride lda elements, cols and lda multiples of 8,
 *   a 16-byte aligned). axis 0: out[c] = max_r |a[r][c]| (out [cols]; the
 *   activation statistic ax[k] over a calibration batch X [M][K]); axis 1:
 *   out[r] = max_c |a[r][c]| (out [rows]; the weight statistic aw[k] of
 *   W [K][N]). accumulate 1 folds the result into the maxima already in
 *   out (calibration over several batches), 0 overwrites them. Inputs are
 *   finite.
 */
svdq_status svdq_calib_absmax(const void* a, int64_t rows, int64_t cols, int64_t lda, int32_t axis,
                              int32_t accumulate, float* out, void* stream);

/* svdq_smoothing -- lambda[k] = ax[k]^alpha / aw[k]^(1 - alpha) in fp64 (1
 *   where either maximum is 0; alpha in [0, 1], 0.5 through square roots),
 *   written as inv_lambda[k] = fp32(1 / lambda[k]) [K]: the online
 *   activation scale (remio.ai page, same section: outliers move into the
 *   weights). */
svdq_status svdq_smoothing(const float* ax, const float* aw, int64_t K, double alpha, float* inv_lambda,
                           void* stream);

/* svdq_smooth_weight -- w_hat[k][n] = f64(W[k][n]) / f64(inv_lambda[k]),
 *   fp64 [K][N] (dense, 16-byte aligned) from bf16 W [K][N] (row stride ldw,
 *   N and ldw multiples of 8, K <= 65535). inv_lambda NULL means 1. */
svdq_status svdq_smooth_weight(const void* w, int64_t K, int64_t N, int64_t ldw, const float* inv_lambda,
                               double* w_hat, void* stream);

/* svdq_lowrank -- the rank-r truncated SVD of w_hat [K][N] (fp64) as the
 *   low-rank branch: L1 = bf16(U_r Sigma_r) [K][r] and L2 = bf16(V_r^T)
 *   [r][N], each entry rounded once from fp64 to nearest even, the entry of
 *   largest magnitude of every right singular vector positive; sigma [r]
 *   (fp64, may be NULL) the singular values, descending. Method: randomised
 *   range finder with power iterations (Halko, Martinsson and Tropp, SIAM
 *   Review 2011, algorithms 4.3/4.4 and 5.1) from the caller's random test
 *   matrix omega [N][l] (fp64, e.g. standard normal), power_iters in
 *   [0, 64], block width l with rank <= l <= min(88, K, N); the l x N
 *   projection is decomposed exactly (Jacobi). rank is a multiple of 16 in
 *   [16, 80]. workspace: device memory of at least
 *   svdq_lowrank_workspace_size() bytes, 256-byte aligned, contents
 *   irrelevant; calls sharing it must not overlap.
 */
svdq_status svdq_lowrank_workspace_size(int64_t K, int64_t N, int32_t rank, int32_t l, int64_t* bytes);
svdq_status svdq_lowrank(const double* w_hat, int64_t K, int64_t N, int32_t rank, const double* omega, int32_t l,
                         int32_t power_iters, void* l1, void* l2, double* sigma, void* workspace,
                         int64_t workspace_bytes, void* stream);

/* svdq_quantize_residual -- R = fp32(w_hat - f64(L1) f64(L2)) (L1 bf16
 *   [K][rank], L2 bf16 [rank][N]; rank a multiple of 16 in [0, 112], 0 = no
 *   branch), then symmetric INT4 per (output column n, group of 64 along
 *   K): s = fp16(min(amax / 7, 65504)), q = clamp(rtne(R * fp32(1 / s)),
 *   -7, 7), all codes 0 where s = 0. Writes qw [N][K/2] (codes format v2)
 *   and sw (scales format v3, [ceil(G/4)][N][4] fp16, padding 0): the
 *   weight operands of svdq_gemm_w4a4. K a multiple of 64; qw 8-byte
 *   aligned. */
svdq_status svdq_quantize_residual(const double* w_hat, int64_t K, int64_t N, const void* l1, const void* l2,
                                   int32_t rank, uint8_t* qw, void* sw_f16, void* stream);

/* svdq_quantize_residual_mxfp4 -- the same residual R as svdq_quantize_residual,
 *   quantised in the MXFP4 layer's number format (OCP Microscaling Formats
 *   v1.0) per output column n and 32-value block along K: E8M0 exponent
 *   e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for a zero block),
 *   codes = E2M1(R * 2^-e) rounded to nearest, ties to mantissa 0, saturating
 *   at 6, zero with sign 0. Writes qw [N][K/2] (E2M1 nibbles, element 2i in
 *   bits 0-3 of byte i; 16-byte aligned) and sw_e8m0, the exponent records
 *   [ceil(K/256)][N][8] (bytes e + 127; block 8q + 2j + h of a column at byte
 *   4h + j of record (q, n); blocks past K hold 0): the weight operands of
 *   svdq_gemm_mxfp4. K a multiple of 64; rank as above. Errors as
 *   svdq_quantize_residual. */
svdq_status svdq_quantize_residual_mxfp4(const double* w_hat, int64_t K, int64_t N, const void* l1, const void* l2,
                                         int32_t rank, uint8_t* qw, uint8_t* sw_e8m0, void* stream);

/* awq_quantize_weight -- the AWQ W4A16 weight quantisation on the GPU, into
 *   the operands of awq_gemv_w4a16 (the textbook asymmetric min/max group
 *   quantiser with the activation-aware channel scale folded into the
 *   weight):
 *   w        bf16 [K][ldw] weight (row k = input channel, N <= ldw columns)
 *   inv_s    fp32 [K] reciprocal channel scales, or NULL (no scaling)
 *   W' = fp32(W / inv_s) (division in fp64, one rounding); per (output
 *   column n, group g of 64 input channels): mn, mx of the group,
 *   s = fp16(max(mx - mn, 1e-5) / 15) in fp32, z = clamp(rtne(-mn * fp32(1 / s)),
 *   0, 15), q = clamp(rtne(W' * fp32(1 / s)) + z, 0, 15).
 *   Writes qwt (codes in the GEMV tile layout, [N/16][K/128][16][64 bytes],
 *   16-byte aligned) and scale_f16 / zero_f16 ([N/16][K/64][16] fp16; z is
 *   an integer). K a positive multiple of 128, N of 16. Errors: shapes ->
 *   SVDQ_ERR_SHAPE, NULL pointers -> SVDQ_ERR_NULL, alignment ->
 *   SVDQ_ERR_ALIGN, no gfx950 device -> SVDQ_ERR_DEVICE. */
svdq_status awq_quantize_weight(const void* w_bf16, int64_t K, int64_t N, int64_t ldw, const float* inv_s,
                                uint8_t* qwt, void* scale_f16, void* zero_f16, void* stream);

/* svdq_pack_lowrank -- L1 [K][rank] and L2 [rank][N] (bf16) into the layouts
 *   the online kernels read: l1t (format v4 tiles, 16-byte aligned) for
 *   svdq_quantize_act and l2t [N][rank] for svdq_gemm_w4a4. rank 0 writes
 *   nothing. */
svdq_status svdq_pack_lowrank(const void* l1, const void* l2, int64_t K, int64_t N, int32_t rank, void* l1t,
                              void* l2t, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
