// Host side of the C ABI declared in include/svdq.h: argument validation
// (before any HIP call), the gfx950 capability check, and kernel launches on
// the caller's stream. No allocation, no synchronisation, no fallback.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/svdq.h"

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            const float* inv_lambda, const uint16_t* l1t, int rank,
                            uint8_t* qx, uint16_t* sx, float* xl1, int cus, hipStream_t stream);
size_t act_quant_smem_bytes(int64_t K, int rank);
hipError_t launch_gemm_w4a4(const uint8_t* qx, const uint16_t* sx, const uint8_t* qw,
                            const uint16_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                            const uint16_t* bias, int act, void* y, int y_f32, int64_t ldy,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_act_quant_mxfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const float* inv_lambda, const uint16_t* l1t, int rank,
                                  uint8_t* qx, uint8_t* sx, float* xl1, int cus, hipStream_t stream);
hipError_t launch_gemm_mxfp4(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw,
                             const uint8_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                             const uint16_t* bias, int act, void* y, int y_f32, int64_t ldy,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_gemm_w4a4_partials(const uint8_t* qx, const uint8_t* qw, int64_t M, int64_t N,
                                     int64_t K, int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                     int32_t* p, hipStream_t stream);
hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t K, const float* inv_s,
                             const uint8_t* qwt, const uint16_t* scale, const uint16_t* zero,
                             int64_t N, const uint16_t* bias, uint16_t* y, int cus, hipStream_t stream);
size_t gemv_smem_bytes(int M, int64_t K);
hipError_t launch_calib_absmax(const uint16_t* a, int64_t rows, int64_t cols, int64_t lda, int axis,
                               int accumulate, float* out, hipStream_t stream);
hipError_t launch_smoothing(const float* ax, const float* aw, int64_t K, double alpha, float* inv_lambda,
                            hipStream_t stream);
hipError_t launch_smooth_weight(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, const float* inv_lambda,
                                double* w_hat, hipStream_t stream);
int64_t offline_lowrank_ws_bytes(int64_t K, int64_t N, int l);
int offline_lmax();
hipError_t launch_lowrank(const double* w_hat, int64_t K, int64_t N, int r, const double* omega, int l,
                          int power_iters, uint16_t* l1, uint16_t* l2, double* sigma, void* ws,
                          hipStream_t stream);
hipError_t launch_quantize_residual(const double* w_hat, int64_t K, int64_t N, const uint16_t* l1,
                                    const uint16_t* l2, int r, uint8_t* qw, uint16_t* sw, hipStream_t stream);
hipError_t launch_quantize_residual_mxfp4(const double* w_hat, int64_t K, int64_t N, const uint16_t* l1,
                                          const uint16_t* l2, int r, uint8_t* qw, uint8_t* se, hipStream_t stream);
hipError_t launch_awq_quantize(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, const float* inv_s,
                               uint8_t* qwt, uint16_t* sc, uint16_t* zr, hipStream_t stream);
hipError_t launch_pack_lowrank(const uint16_t* l1, const uint16_t* l2, int64_t K, int64_t N, int r, uint16_t* l1t,
                               uint16_t* l2t, hipStream_t stream);
int64_t gemm_next_partial_bytes(int64_t M, int64_t N, int rank_next);
hipError_t launch_gemm_w4a4_next(const uint8_t* qx, const uint16_t* sx, const uint8_t* qw,
                                 const uint16_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                                 const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                                 const float* inv_next, const uint16_t* l1t_next, int rank_next,
                                 uint8_t* qx_next, uint16_t* sx_next, float* xl1_next, float* part,
                                 hipStream_t stream, int fmt);
hipError_t launch_clock_probe(long long* out, int spins, hipStream_t stream);
hipError_t launch_read_probe(const uint8_t* buf, int64_t bytes, uint32_t* sink, int blocks,
                             hipStream_t stream);

namespace {

constexpr size_t kMaxLds = 160 * 1024;   // LDS per CU on gfx950

thread_local std::string g_last_error;

svdq_status fail(svdq_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Per-device capability cache: 0 = unknown, 1 = gfx950, 2 = not supported;
// and the device's compute-unit count (persistent grids).
constexpr int kMaxDev = 64;
int g_dev_ok[kMaxDev];
int g_dev_cus[kMaxDev];
std::mutex g_dev_mu;

svdq_status check_device_id(int dev) {
    if (dev < 0 || dev >= kMaxDev) return fail(SVDQ_ERR_DEVICE, "device %d out of range", dev);
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_ok[dev] == 1) return SVDQ_OK;
        if (g_dev_ok[dev] == 2) return fail(SVDQ_ERR_DEVICE, "device %d is not gfx950", dev);
    }
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(SVDQ_ERR_DEVICE, "no HIP device is available");
    }
    if (dev >= count) return fail(SVDQ_ERR_DEVICE, "device %d does not exist (%d present)", dev, count);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(SVDQ_ERR_DEVICE, "cannot query device %d", dev);
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        g_dev_ok[dev] = ok ? 1 : 2;
        g_dev_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    }
    if (!ok) return fail(SVDQ_ERR_DEVICE, "device %d is %s, these kernels are built for gfx950 only",
                         dev, prop.gcnArchName);
    return SVDQ_OK;
}

svdq_status check_current_device(int* cus = nullptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(SVDQ_ERR_DEVICE, "no current HIP device");
    }
    const svdq_status s = check_device_id(dev);
    if (s == SVDQ_OK && cus) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        *cus = g_dev_cus[dev];
    }
    return s;
}

svdq_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    g_last_error.clear();
    return SVDQ_OK;
}

svdq_status check_rank(int32_t rank) {
    if (rank < 0 || rank > 128 || rank % 16 != 0)
        return fail(SVDQ_ERR_SHAPE, "rank %d must be a multiple of 16 in [0, 128]", rank);
    return SVDQ_OK;
}

svdq_status check_n(int64_t N) {
    if (N <= 0 || N % 8) return fail(SVDQ_ERR_SHAPE, "N = %lld must be a positive multiple of 8", (long long)N);
    if (N > ((int64_t)1 << 31)) return fail(SVDQ_ERR_SHAPE, "N = %lld too large", (long long)N);
    return SVDQ_OK;
}

svdq_status check_act(int32_t act) {
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_UNSUPPORTED, "activation %d is not supported", act);
    return SVDQ_OK;
}

svdq_status check_k(int64_t K) {
    if (K <= 0 || K % 64 != 0) return fail(SVDQ_ERR_SHAPE, "K = %lld must be a positive multiple of 64", (long long)K);
    if (K > (int64_t)1 << 30) return fail(SVDQ_ERR_SHAPE, "K = %lld too large", (long long)K);
    return SVDQ_OK;
}

// the GEMM addresses the packed codes and scales with 31-bit byte offsets,
// including rows up to one tile past the end of the matrix
svdq_status check_gemm_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t lim = (int64_t)1 << 31;
    if ((M + 256) * (K / 2) >= lim || (N + 256) * (K / 2) >= lim)
        return fail(SVDQ_ERR_SHAPE, "(M + 256) * K / 2 and (N + 256) * K / 2 must stay below 2^31 bytes");
    return SVDQ_OK;
}

svdq_status quantize_act_impl(int mxfp4, const void* x, int64_t M, int64_t K, int64_t ldx,
                              const float* inv_lambda, const void* l1t, int32_t rank,
                              uint8_t* qx, void* sx_f16, float* xl1, void* stream) {
    svdq_status s;
    if (M < 0) return fail(SVDQ_ERR_SHAPE, "M = %lld is negative", (long long)M);
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if ((s = check_rank(rank)) != SVDQ_OK) return s;
    if (ldx < K) return fail(SVDQ_ERR_SHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
    if (ldx % 8) return fail(SVDQ_ERR_ALIGN, "ldx = %lld must be a multiple of 8", (long long)ldx);
    if (ldx >= ((int64_t)1 << 26))
        return fail(SVDQ_ERR_SHAPE, "ldx = %lld must be below 2^26 (16 rows addressed with 31-bit offsets)",
                    (long long)ldx);
    if (act_quant_smem_bytes(K, rank) > kMaxLds)
        return fail(SVDQ_ERR_SHAPE, "K = %lld with rank %d exceeds the LDS budget", (long long)K, rank);
    if (M == 0) { g_last_error.clear(); return SVDQ_OK; }   // empty batch: nothing to read or write
    if (!x || !qx || !sx_f16) return fail(SVDQ_ERR_NULL, "x, qx and sx_f16 are required");
    if (rank > 0 && (!l1t || !xl1)) return fail(SVDQ_ERR_NULL, "rank %d needs l1t and xl1", rank);
    if (!aligned(x, 16) || !aligned(qx, 16) || !aligned(sx_f16, 16) ||
        (inv_lambda && !aligned(inv_lambda, 16)) ||
        (rank > 0 && (!aligned(l1t, 16) || !aligned(xl1, 16))))
        return fail(SVDQ_ERR_ALIGN, "x, inv_lambda, l1t, qx, sx_f16, xl1 need 16-byte alignment");
    int cus = 0;
    if ((s = check_current_device(&cus)) != SVDQ_OK) return s;
    const uint16_t* l1 = rank > 0 ? (const uint16_t*)l1t : nullptr;
    float* xo = rank > 0 ? xl1 : nullptr;
    if (mxfp4)
        return launched(launch_act_quant_mxfp4((const uint16_t*)x, M, K, ldx, inv_lambda, l1, rank, qx,
                                               (uint8_t*)sx_f16, xo, cus, (hipStream_t)stream),
                        "svdq_quantize_act_mxfp4 launch");
    return launched(launch_act_quant((const uint16_t*)x, M, K, ldx, inv_lambda, l1, rank, qx,
                                     (uint16_t*)sx_f16, xo, cus, (hipStream_t)stream),
                    "svdq_quantize_act launch");
}

svdq_status gemm_impl(int mxfp4, const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                           const uint8_t* qw, const void* sw_f16, int64_t N,
                           const float* xl1, const void* l2t, int32_t rank,
                           const void* bias, int32_t act,
                           void* y, int32_t y_dtype, int64_t ldy, void* stream) {
    svdq_status s;
    if (M < 0) return fail(SVDQ_ERR_SHAPE, "M = %lld is negative", (long long)M);
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if ((s = check_rank(rank)) != SVDQ_OK) return s;
    if ((s = check_n(N)) != SVDQ_OK) return s;
    if (M > ((int64_t)1 << 31)) return fail(SVDQ_ERR_SHAPE, "M = %lld too large", (long long)M);
    if ((s = check_gemm_bytes(M, N, K)) != SVDQ_OK) return s;
    if ((M + 256) * rank * 4 >= ((int64_t)1 << 31) || (N + 256) * rank * 2 >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "(M + 256) * rank * 4 and (N + 256) * rank * 2 must stay below 2^31 bytes");
    if (ldy < N) return fail(SVDQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
    if (ldy % 8) return fail(SVDQ_ERR_ALIGN, "ldy = %lld must be a multiple of 8", (long long)ldy);
    if ((M + 128) * ldy * (y_dtype == SVDQ_DT_F32 ? 4 : 2) >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "(M + 128) * ldy * element size must stay below 2^31 bytes");
    if ((s = check_act(act)) != SVDQ_OK) return s;
    if (y_dtype != SVDQ_DT_BF16 && y_dtype != SVDQ_DT_F32)
        return fail(SVDQ_ERR_UNSUPPORTED, "output dtype %d is not supported", y_dtype);
    if (M == 0) { g_last_error.clear(); return SVDQ_OK; }   // empty batch
    if (!qx || !sx_f16 || !qw || !sw_f16 || !y) return fail(SVDQ_ERR_NULL, "qx, sx, qw, sw and y are required");
    if (rank > 0 && (!xl1 || !l2t)) return fail(SVDQ_ERR_NULL, "rank %d needs xl1 and l2t", rank);
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(y, 16) || !aligned(sx_f16, 16) ||
        !aligned(sw_f16, 16) || (bias && !aligned(bias, 2)) ||
        (rank > 0 && (!aligned(xl1, 16) || !aligned(l2t, 16))))
        return fail(SVDQ_ERR_ALIGN, "qx, sx, qw, sw, xl1, l2t, y need 16-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    const float* xo = rank > 0 ? xl1 : nullptr;
    const uint16_t* l2 = rank > 0 ? (const uint16_t*)l2t : nullptr;
    if (mxfp4)
        return launched(launch_gemm_mxfp4(qx, (const uint8_t*)sx_f16, qw, (const uint8_t*)sw_f16, xo, l2,
                                          rank, (const uint16_t*)bias, act, y, y_dtype == SVDQ_DT_F32, ldy,
                                          M, N, K, (hipStream_t)stream),
                        "svdq_gemm_mxfp4 launch");
    return launched(launch_gemm_w4a4(qx, (const uint16_t*)sx_f16, qw, (const uint16_t*)sw_f16, xo, l2,
                                     rank, (const uint16_t*)bias, act, y, y_dtype == SVDQ_DT_F32, ldy,
                                     M, N, K, (hipStream_t)stream),
                    "svdq_gemm_w4a4 launch");
}

svdq_status validate_desc(const svdq_layer_desc* d) {
    svdq_status s;
    if (!d) return fail(SVDQ_ERR_NULL, "layer description is NULL");
    if ((s = check_k(d->K)) != SVDQ_OK) return s;
    if ((s = check_n(d->N)) != SVDQ_OK) return s;
    if ((s = check_rank(d->rank)) != SVDQ_OK) return s;
    if (d->group != 64) return fail(SVDQ_ERR_UNSUPPORTED, "group size %d is not supported (only 64)", d->group);
    if (d->fmt != SVDQ_FMT_INT4 && d->fmt != SVDQ_FMT_MXFP4)
        return fail(SVDQ_ERR_UNSUPPORTED, "format %d is not supported (0 = INT4, 1 = MXFP4)", d->fmt);
    if ((s = check_act(d->act)) != SVDQ_OK) return s;
    if ((s = check_gemm_bytes(0, d->N, d->K)) != SVDQ_OK) return s;
    g_last_error.clear();
    return SVDQ_OK;
}

}  // namespace

extern "C" {

svdq_status svdq_validate_desc(const svdq_layer_desc* desc) { return validate_desc(desc); }

svdq_status svdq_layer_sizes_of(const svdq_layer_desc* d, svdq_layer_sizes* out) {
    svdq_status s;
    if ((s = validate_desc(d)) != SVDQ_OK) return s;
    if (!out) return fail(SVDQ_ERR_NULL, "sizes is NULL");
    const int64_t G4 = (d->K / 64 + 3) / 4;
    out->qw = d->N * (d->K / 2);
    out->sw = G4 * d->N * 8;              // 4 fp16 or 8 E8M0 bytes per (quad, row)
    out->l1t = d->K * d->rank * 2;
    out->l2t = d->N * d->rank * 2;
    out->inv_lambda = d->K * 4;
    out->bias = d->N * 2;
    out->qx_row = d->K / 2;
    out->sx_row = G4 * 8;
    out->xl1_row = (int64_t)d->rank * 4;
    return SVDQ_OK;
}

const char* svdq_status_string(svdq_status s) {
    switch (s) {
        case SVDQ_OK: return "ok";
        case SVDQ_ERR_NULL: return "null pointer";
        case SVDQ_ERR_SHAPE: return "invalid shape";
        case SVDQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case SVDQ_ERR_UNSUPPORTED: return "unsupported option";
        case SVDQ_ERR_DEVICE: return "unsupported or missing device";
        case SVDQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* svdq_last_error(void) { return g_last_error.c_str(); }

int svdq_version(void) { return 404; }

svdq_status svdq_check_device(int device) {
    svdq_status s = check_device_id(device);
    if (s == SVDQ_OK) g_last_error.clear();
    return s;
}

svdq_status svdq_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx,
                              const float* inv_lambda, const void* l1t, int32_t rank,
                              uint8_t* qx, void* sx_f16, float* xl1, void* stream) {
    return quantize_act_impl(0, x, M, K, ldx, inv_lambda, l1t, rank, qx, sx_f16, xl1, stream);
}

svdq_status svdq_quantize_act_mxfp4(const void* x, int64_t M, int64_t K, int64_t ldx,
                                    const float* inv_lambda, const void* l1t, int32_t rank,
                                    uint8_t* qx, void* sx_e8m0, float* xl1, void* stream) {
    return quantize_act_impl(1, x, M, K, ldx, inv_lambda, l1t, rank, qx, sx_e8m0, xl1, stream);
}

svdq_status svdq_gemm_w4a4(const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                           const uint8_t* qw, const void* sw_f16, int64_t N,
                           const float* xl1, const void* l2t, int32_t rank,
                           const void* bias, int32_t act,
                           void* y, int32_t y_dtype, int64_t ldy, void* stream) {
    return gemm_impl(0, qx, sx_f16, M, K, qw, sw_f16, N, xl1, l2t, rank, bias, act, y, y_dtype, ldy, stream);
}

svdq_status svdq_gemm_mxfp4(const uint8_t* qx, const void* sx_e8m0, int64_t M, int64_t K,
                            const uint8_t* qw, const void* sw_e8m0, int64_t N,
                            const float* xl1, const void* l2t, int32_t rank,
                            const void* bias, int32_t act,
                            void* y, int32_t y_dtype, int64_t ldy, void* stream) {
    return gemm_impl(1, qx, sx_e8m0, M, K, qw, sw_e8m0, N, xl1, l2t, rank, bias, act, y, y_dtype, ldy, stream);
}

svdq_status svdq_gemm_w4a4_partials(const uint8_t* qx, int64_t M, int64_t K,
                                    const uint8_t* qw, int64_t N,
                                    int64_t m0, int64_t mcount, int64_t n0, int64_t ncount,
                                    int32_t* p, void* stream) {
    svdq_status s;
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if (M < 0 || N <= 0 || N % 8) return fail(SVDQ_ERR_SHAPE, "bad M or N");
    if ((s = check_gemm_bytes(M, N, K)) != SVDQ_OK) return s;
    if (m0 < 0 || mcount < 0 || m0 + mcount > M || n0 < 0 || ncount < 0 || n0 + ncount > N)
        return fail(SVDQ_ERR_SHAPE, "rectangle outside the M x N output");
    if (mcount == 0 || ncount == 0) { g_last_error.clear(); return SVDQ_OK; }
    if (!qx || !qw || !p) return fail(SVDQ_ERR_NULL, "qx, qw and p are required");
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(p, 4))
        return fail(SVDQ_ERR_ALIGN, "qx, qw need 16-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_gemm_w4a4_partials(qx, qw, M, N, K, m0, mcount, n0, ncount, p,
                                              (hipStream_t)stream),
                    "svdq_gemm_w4a4_partials launch");
}

svdq_status awq_gemv_w4a16(const void* x, int64_t M, int64_t K, const float* inv_s,
                           const uint8_t* qwt, const void* scale_f16, const void* zero_f16,
                           int64_t N, const void* bias, void* y, void* stream) {
    const uint8_t* qw = qwt;
    svdq_status s;
    if (M < 1 || M > 16) return fail(SVDQ_ERR_SHAPE, "M = %lld must be in [1, 16]", (long long)M);
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if (K % 128) return fail(SVDQ_ERR_SHAPE, "K = %lld must be a multiple of 128 (group pairs)", (long long)K);
    if (N <= 0 || N % 16) return fail(SVDQ_ERR_SHAPE, "N = %lld must be a positive multiple of 16", (long long)N);
    // the kernel addresses every array with 31-bit byte offsets
    const int64_t lim = (int64_t)1 << 31;
    if (N * (K / 2) >= lim || N * (K / 64) * 2 >= lim || M * K * 2 >= lim || K * 4 >= lim)
        return fail(SVDQ_ERR_SHAPE, "N = %lld, K = %lld: packed weights or scales exceed 2 GiB",
                    (long long)N, (long long)K);
    if (!x || !qw || !scale_f16 || !zero_f16 || !y) return fail(SVDQ_ERR_NULL, "x, qw, scale, zero and y are required");
    if (!aligned(x, 16) || !aligned(qw, 16) || !aligned(y, 16) || !aligned(scale_f16, 2) ||
        !aligned(zero_f16, 2) || (inv_s && !aligned(inv_s, 16)) || (bias && !aligned(bias, 2)))
        return fail(SVDQ_ERR_ALIGN, "x, inv_s, qw, y need 16-byte alignment, scale/zero 2 bytes");
    if (gemv_smem_bytes((int)M, K) > kMaxLds) return fail(SVDQ_ERR_SHAPE, "M too large for the LDS budget");
    int cus = 0;
    if ((s = check_current_device(&cus)) != SVDQ_OK) return s;
    return launched(launch_gemv_w4a16((const uint16_t*)x, (int)M, K, inv_s, qw,
                                      (const uint16_t*)scale_f16, (const uint16_t*)zero_f16, N,
                                      (const uint16_t*)bias, (uint16_t*)y, cus, (hipStream_t)stream),
                    "awq_gemv_w4a16 launch");
}

svdq_status svdq_probe_clock(int64_t* ticks, int32_t spins, void* stream) {
    svdq_status s;
    if (spins < 1 || spins > 10000000) return fail(SVDQ_ERR_SHAPE, "spins = %d must be in [1, 1e7]", spins);
    if (!ticks) return fail(SVDQ_ERR_NULL, "ticks is required");
    if (!aligned(ticks, 8)) return fail(SVDQ_ERR_ALIGN, "ticks needs 8-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_clock_probe((long long*)ticks, spins, (hipStream_t)stream), "svdq_probe_clock launch");
}

svdq_status svdq_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
    svdq_status s;
    if (bytes <= 0 || bytes % 16 || bytes >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "bytes = %lld must be a positive multiple of 16 below 2^31", (long long)bytes);
    if (blocks < 1 || blocks > 65536) return fail(SVDQ_ERR_SHAPE, "blocks = %d must be in [1, 65536]", blocks);
    if (!buf || !sink) return fail(SVDQ_ERR_NULL, "buf and sink are required");
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(SVDQ_ERR_ALIGN, "buf needs 16-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_read_probe((const uint8_t*)buf, bytes, sink, blocks, (hipStream_t)stream),
                    "svdq_probe_read launch");
}

}  // extern "C"

/* ------------------------------------------------------------------------ */
/* offline quantiser                                                         */

namespace {

// element counts the offline kernels index with 64-bit offsets; a product of
// two sizes must stay far from overflow
svdq_status check_dims(int64_t a, int64_t b, const char* what) {
    if (a < 0 || b < 0 || (a > 0 && b > (((int64_t)1 << 46) / a)))
        return fail(SVDQ_ERR_SHAPE, "%s: %lld x %lld is out of range", what, (long long)a, (long long)b);
    return SVDQ_OK;
}

}  // namespace

svdq_status svdq_calib_absmax(const void* a, int64_t rows, int64_t cols, int64_t lda, int32_t axis,
                              int32_t accumulate, float* out, void* stream) {
    svdq_status s;
    if (axis != 0 && axis != 1) return fail(SVDQ_ERR_UNSUPPORTED, "axis %d must be 0 or 1", axis);
    if (accumulate != 0 && accumulate != 1) return fail(SVDQ_ERR_UNSUPPORTED, "accumulate must be 0 or 1");
    if ((s = check_dims(rows, cols, "svdq_calib_absmax")) != SVDQ_OK) return s;
    if (cols % 8) return fail(SVDQ_ERR_SHAPE, "cols = %lld must be a multiple of 8", (long long)cols);
    if (lda < cols || lda % 8) return fail(SVDQ_ERR_SHAPE, "lda = %lld must be >= cols and a multiple of 8", (long long)lda);
    const int64_t n = axis == 0 ? cols : rows;
    if (n == 0) { g_last_error.clear(); return SVDQ_OK; }
    if (!out || (rows > 0 && cols > 0 && !a)) return fail(SVDQ_ERR_NULL, "a and out are required");
    if ((a && !aligned(a, 16)) || !aligned(out, 4)) return fail(SVDQ_ERR_ALIGN, "a needs 16-byte alignment, out 4");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_calib_absmax((const uint16_t*)a, rows, cols, lda, axis, accumulate, out,
                                        (hipStream_t)stream),
                    "svdq_calib_absmax launch");
}

svdq_status svdq_smoothing(const float* ax, const float* aw, int64_t K, double alpha, float* inv_lambda,
                           void* stream) {
    svdq_status s;
    if (K < 0) return fail(SVDQ_ERR_SHAPE, "K = %lld must be >= 0", (long long)K);
    if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(SVDQ_ERR_UNSUPPORTED, "alpha %g must be in [0, 1]", alpha);
    if (K == 0) { g_last_error.clear(); return SVDQ_OK; }
    if (!ax || !aw || !inv_lambda) return fail(SVDQ_ERR_NULL, "ax, aw and inv_lambda are required");
    if (!aligned(ax, 4) || !aligned(aw, 4) || !aligned(inv_lambda, 4)) return fail(SVDQ_ERR_ALIGN, "4-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_smoothing(ax, aw, K, alpha, inv_lambda, (hipStream_t)stream), "svdq_smoothing launch");
}

svdq_status svdq_smooth_weight(const void* w, int64_t K, int64_t N, int64_t ldw, const float* inv_lambda,
                               double* w_hat, void* stream) {
    svdq_status s;
    if ((s = check_dims(K, N, "svdq_smooth_weight")) != SVDQ_OK) return s;
    if (K > 65535) return fail(SVDQ_ERR_SHAPE, "K = %lld above 65535", (long long)K);
    if (N % 8) return fail(SVDQ_ERR_SHAPE, "N = %lld must be a multiple of 8", (long long)N);
    if (ldw < N || ldw % 8) return fail(SVDQ_ERR_SHAPE, "ldw = %lld must be >= N and a multiple of 8", (long long)ldw);
    if (K == 0 || N == 0) { g_last_error.clear(); return SVDQ_OK; }
    if (!w || !w_hat) return fail(SVDQ_ERR_NULL, "w and w_hat are required");
    if (!aligned(w, 16) || !aligned(w_hat, 16) || (inv_lambda && !aligned(inv_lambda, 4)))
        return fail(SVDQ_ERR_ALIGN, "w and w_hat need 16-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_smooth_weight((const uint16_t*)w, K, N, ldw, inv_lambda, w_hat, (hipStream_t)stream),
                    "svdq_smooth_weight launch");
}

namespace {

svdq_status check_lowrank_shape(int64_t K, int64_t N, int32_t rank, int32_t l) {
    svdq_status s;
    if ((s = check_dims(K, N, "svdq_lowrank")) != SVDQ_OK) return s;
    if (K < 1 || N < 1) return fail(SVDQ_ERR_SHAPE, "K and N must be >= 1");
    if (rank < 1 || rank > 80 || rank % 16)
        return fail(SVDQ_ERR_SHAPE, "rank %d must be a multiple of 16 in [16, 80]", rank);
    const int64_t mn = K < N ? K : N;
    if (l < rank || l > offline_lmax() || l > mn)
        return fail(SVDQ_ERR_SHAPE, "block width l = %d must satisfy rank <= l <= min(%d, K, N)", l, offline_lmax());
    return SVDQ_OK;
}

}  // namespace

svdq_status svdq_lowrank_workspace_size(int64_t K, int64_t N, int32_t rank, int32_t l, int64_t* bytes) {
    svdq_status s;
    if (!bytes) return fail(SVDQ_ERR_NULL, "bytes is required");
    if ((s = check_lowrank_shape(K, N, rank, l)) != SVDQ_OK) return s;
    *bytes = offline_lowrank_ws_bytes(K, N, l);
    g_last_error.clear();
    return SVDQ_OK;
}

svdq_status svdq_lowrank(const double* w_hat, int64_t K, int64_t N, int32_t rank, const double* omega, int32_t l,
                         int32_t power_iters, void* l1, void* l2, double* sigma, void* workspace,
                         int64_t workspace_bytes, void* stream) {
    svdq_status s;
    if ((s = check_lowrank_shape(K, N, rank, l)) != SVDQ_OK) return s;
    if (power_iters < 0 || power_iters > 64) return fail(SVDQ_ERR_SHAPE, "power_iters %d must be in [0, 64]", power_iters);
    if (workspace_bytes < offline_lowrank_ws_bytes(K, N, l))
        return fail(SVDQ_ERR_SHAPE, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)offline_lowrank_ws_bytes(K, N, l));
    if (!w_hat || !omega || !l1 || !l2 || !workspace) return fail(SVDQ_ERR_NULL, "w_hat, omega, l1, l2, workspace are required");
    if (!aligned(w_hat, 8) || !aligned(omega, 8) || !aligned(l1, 2) || !aligned(l2, 2) ||
        (sigma && !aligned(sigma, 8)) || !aligned(workspace, 256))
        return fail(SVDQ_ERR_ALIGN, "w_hat, omega, sigma 8-byte, l1, l2 2-byte, workspace 256-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_lowrank(w_hat, K, N, rank, omega, l, power_iters, (uint16_t*)l1, (uint16_t*)l2, sigma,
                                   workspace, (hipStream_t)stream),
                    "svdq_lowrank launch");
}

svdq_status svdq_quantize_residual(const double* w_hat, int64_t K, int64_t N, const void* l1, const void* l2,
                                   int32_t rank, uint8_t* qw, void* sw_f16, void* stream) {
    svdq_status s;
    if ((s = check_dims(K, N, "svdq_quantize_residual")) != SVDQ_OK) return s;
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if (K / 64 > 65535) return fail(SVDQ_ERR_SHAPE, "K = %lld: more than 65535 groups", (long long)K);
    if (N < 1) return fail(SVDQ_ERR_SHAPE, "N must be >= 1");
    if (rank < 0 || rank > 112 || rank % 16) return fail(SVDQ_ERR_SHAPE, "rank %d must be a multiple of 16 in [0, 112]", rank);
    if (!w_hat || !qw || !sw_f16 || (rank > 0 && (!l1 || !l2)))
        return fail(SVDQ_ERR_NULL, "w_hat, qw, sw (and l1, l2 when rank > 0) are required");
    if (!aligned(w_hat, 8) || !aligned(qw, 8) || !aligned(sw_f16, 2) || (l1 && !aligned(l1, 2)) || (l2 && !aligned(l2, 2)))
        return fail(SVDQ_ERR_ALIGN, "w_hat, qw 8-byte, sw, l1, l2 2-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_quantize_residual(w_hat, K, N, (const uint16_t*)l1, (const uint16_t*)l2, rank, qw,
                                             (uint16_t*)sw_f16, (hipStream_t)stream),
                    "svdq_quantize_residual launch");
}

svdq_status svdq_quantize_residual_mxfp4(const double* w_hat, int64_t K, int64_t N, const void* l1, const void* l2,
                                         int32_t rank, uint8_t* qw, uint8_t* sw_e8m0, void* stream) {
    svdq_status s;
    if ((s = check_dims(K, N, "svdq_quantize_residual_mxfp4")) != SVDQ_OK) return s;
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if (K / 64 > 65535) return fail(SVDQ_ERR_SHAPE, "K = %lld: more than 65535 groups", (long long)K);
    if (N < 1) return fail(SVDQ_ERR_SHAPE, "N must be >= 1");
    if (rank < 0 || rank > 112 || rank % 16) return fail(SVDQ_ERR_SHAPE, "rank %d must be a multiple of 16 in [0, 112]", rank);
    if (!w_hat || !qw || !sw_e8m0 || (rank > 0 && (!l1 || !l2)))
        return fail(SVDQ_ERR_NULL, "w_hat, qw, sw (and l1, l2 when rank > 0) are required");
    if (!aligned(w_hat, 8) || !aligned(qw, 16) || (l1 && !aligned(l1, 2)) || (l2 && !aligned(l2, 2)))
        return fail(SVDQ_ERR_ALIGN, "w_hat 8-byte, qw 16-byte, l1, l2 2-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_quantize_residual_mxfp4(w_hat, K, N, (const uint16_t*)l1, (const uint16_t*)l2, rank, qw,
                                                   sw_e8m0, (hipStream_t)stream),
                    "svdq_quantize_residual_mxfp4 launch");
}

svdq_status awq_quantize_weight(const void* w_bf16, int64_t K, int64_t N, int64_t ldw, const float* inv_s,
                                uint8_t* qwt, void* scale_f16, void* zero_f16, void* stream) {
    svdq_status s;
    if (K < 128 || K % 128) return fail(SVDQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128", (long long)K);
    if (N < 16 || N % 16) return fail(SVDQ_ERR_SHAPE, "N = %lld must be a positive multiple of 16", (long long)N);
    if (ldw < N) return fail(SVDQ_ERR_SHAPE, "ldw = %lld is below N = %lld", (long long)ldw, (long long)N);
    if (K / 64 > 65535) return fail(SVDQ_ERR_SHAPE, "K = %lld: more than 65535 groups", (long long)K);
    if (!w_bf16 || !qwt || !scale_f16 || !zero_f16) return fail(SVDQ_ERR_NULL, "w, qwt, scale and zero are required");
    if (!aligned(w_bf16, 2) || !aligned(qwt, 16) || !aligned(scale_f16, 2) || !aligned(zero_f16, 2) ||
        (inv_s && !aligned(inv_s, 4)))
        return fail(SVDQ_ERR_ALIGN, "qwt needs 16-byte alignment, inv_s 4, w, scale and zero 2");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_awq_quantize((const uint16_t*)w_bf16, K, N, ldw, inv_s, qwt, (uint16_t*)scale_f16,
                                        (uint16_t*)zero_f16, (hipStream_t)stream),
                    "awq_quantize_weight launch");
}

svdq_status svdq_pack_lowrank(const void* l1, const void* l2, int64_t K, int64_t N, int32_t rank, void* l1t,
                              void* l2t, void* stream) {
    svdq_status s;
    if ((s = check_dims(K, N, "svdq_pack_lowrank")) != SVDQ_OK) return s;
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if ((s = check_rank(rank)) != SVDQ_OK) return s;
    if (N < 1) return fail(SVDQ_ERR_SHAPE, "N must be >= 1");
    if (rank == 0) { g_last_error.clear(); return SVDQ_OK; }
    if (!l1 || !l2 || !l1t || !l2t) return fail(SVDQ_ERR_NULL, "l1, l2, l1t, l2t are required");
    if (!aligned(l1, 2) || !aligned(l2, 2) || !aligned(l1t, 16) || !aligned(l2t, 2))
        return fail(SVDQ_ERR_ALIGN, "l1t needs 16-byte alignment, the others 2");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_pack_lowrank((const uint16_t*)l1, (const uint16_t*)l2, K, N, rank, (uint16_t*)l1t,
                                        (uint16_t*)l2t, (hipStream_t)stream),
                    "svdq_pack_lowrank launch");
}

/* ------------------------------------------------------------------------ */
/* GEMM with the next layer's activation pass in its epilogue                 */

namespace {

svdq_status check_next_shape(int64_t M, int64_t N, int32_t rank_next) {
    if (M < 0) return fail(SVDQ_ERR_SHAPE, "M = %lld must be >= 0", (long long)M);
    if (N <= 0 || N % 128) return fail(SVDQ_ERR_SHAPE, "N = %lld must be a positive multiple of 128 (whole tiles)", (long long)N);
    if (rank_next < 0 || rank_next > 64 || rank_next % 16)
        return fail(SVDQ_ERR_SHAPE, "rank_next %d must be a multiple of 16 in [0, 64]", rank_next);
    if ((N / 128) * M * rank_next * 4 >= ((int64_t)1 << 40)) return fail(SVDQ_ERR_SHAPE, "partials too large");
    return SVDQ_OK;
}

}  // namespace

svdq_status svdq_gemm_w4a4_quant_next_workspace_size(int64_t M, int64_t N, int32_t rank_next, int64_t* bytes) {
    svdq_status s;
    if (!bytes) return fail(SVDQ_ERR_NULL, "bytes is required");
    if ((s = check_next_shape(M, N, rank_next)) != SVDQ_OK) return s;
    *bytes = gemm_next_partial_bytes(M, N, rank_next);
    g_last_error.clear();
    return SVDQ_OK;
}

namespace {

// both formats: the checks, then the launch (fmt 0 INT4, 1 MXFP4)
svdq_status gemm_quant_next(const char* fn, int fmt, const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                                      const uint8_t* qw, const void* sw_f16, int64_t N,
                                      const float* xl1, const void* l2t, int32_t rank,
                                      const void* bias, int32_t act,
                                      const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                      uint8_t* qx_next, void* sx_next_f16, float* xl1_next,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
    svdq_status s;
    if ((s = check_k(K)) != SVDQ_OK) return s;
    if ((s = check_rank(rank)) != SVDQ_OK) return s;
    if ((s = check_act(act)) != SVDQ_OK) return s;
    if ((s = check_next_shape(M, N, rank_next)) != SVDQ_OK) return s;
    if ((s = check_gemm_bytes(M, N, K)) != SVDQ_OK) return s;
    if ((M + 256) * rank * 4 >= ((int64_t)1 << 31) || (N + 256) * rank * 2 >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "(M + 256) * rank * 4 and (N + 256) * rank * 2 must stay below 2^31 bytes");
    if (M * (N / 2) >= ((int64_t)1 << 31) || rank_next * N * 2 >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "the next layer's codes or L1 exceed 2 GiB");
    if (M == 0) { g_last_error.clear(); return SVDQ_OK; }
    if (!qx || !sx_f16 || !qw || !sw_f16 || !inv_lambda_next || !qx_next || !sx_next_f16)
        return fail(SVDQ_ERR_NULL, "qx, sx, qw, sw, inv_lambda_next, qx_next and sx_next are required");
    if (rank > 0 && (!xl1 || !l2t)) return fail(SVDQ_ERR_NULL, "xl1 and l2t are required when rank > 0");
    if (rank_next > 0 && (!l1t_next || !xl1_next || !workspace))
        return fail(SVDQ_ERR_NULL, "l1t_next, xl1_next and workspace are required when rank_next > 0");
    if (rank_next > 0 && workspace_bytes < gemm_next_partial_bytes(M, N, rank_next))
        return fail(SVDQ_ERR_SHAPE, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)gemm_next_partial_bytes(M, N, rank_next));
    if (!aligned(qx, 16) || !aligned(qw, 16) || !aligned(sx_f16, 16) || !aligned(sw_f16, 16) ||
        (xl1 && !aligned(xl1, 16)) || (l2t && !aligned(l2t, 16)) || (bias && !aligned(bias, 2)) ||
        !aligned(inv_lambda_next, 16) || (l1t_next && !aligned(l1t_next, 16)) || !aligned(qx_next, 16) ||
        !aligned(sx_next_f16, fmt == 1 ? 1 : 2) || (xl1_next && !aligned(xl1_next, 16)) ||
        (workspace && !aligned(workspace, 16)))
        return fail(SVDQ_ERR_ALIGN, "vector operands need 16-byte alignment (sx_next %d, bias 2)", fmt == 1 ? 1 : 2);
    if ((s = check_current_device()) != SVDQ_OK) return s;
    return launched(launch_gemm_w4a4_next(qx, (const uint16_t*)sx_f16, qw, (const uint16_t*)sw_f16, xl1,
                                          (const uint16_t*)l2t, rank, (const uint16_t*)bias, act, M, N, K,
                                          inv_lambda_next, (const uint16_t*)l1t_next, rank_next, qx_next,
                                          (uint16_t*)sx_next_f16, xl1_next, (float*)workspace, (hipStream_t)stream,
                                          fmt),
                    fn);
}

}  // namespace

svdq_status svdq_gemm_w4a4_quant_next(const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                                      const uint8_t* qw, const void* sw_f16, int64_t N,
                                      const float* xl1, const void* l2t, int32_t rank,
                                      const void* bias, int32_t act,
                                      const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                      uint8_t* qx_next, void* sx_next_f16, float* xl1_next,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
    return gemm_quant_next("svdq_gemm_w4a4_quant_next launch", 0, qx, sx_f16, M, K, qw, sw_f16, N, xl1, l2t, rank,
                           bias, act, inv_lambda_next, l1t_next, rank_next, qx_next, sx_next_f16, xl1_next,
                           workspace, workspace_bytes, stream);
}

svdq_status svdq_gemm_mxfp4_quant_next(const uint8_t* qx, const void* sx, int64_t M, int64_t K,
                                       const uint8_t* qw, const void* sw, int64_t N,
                                       const float* xl1, const void* l2t, int32_t rank,
                                       const void* bias, int32_t act,
                                       const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                       uint8_t* qx_next, void* sx_next, float* xl1_next,
                                       void* workspace, int64_t workspace_bytes, void* stream) {
    return gemm_quant_next("svdq_gemm_mxfp4_quant_next launch", 1, qx, sx, M, K, qw, sw, N, xl1, l2t, rank,
                           bias, act, inv_lambda_next, l1t_next, rank_next, qx_next, sx_next, xl1_next,
                           workspace, workspace_bytes, stream);
}

/* ------------------------------------------------------------------------ */
/* allocation-free form of svdq_gemm_w4a4_quant_next                          */

namespace {

// The tile partials of svdq_gemm_w4a4_quant_next_noalloc live here: one copy
// per GPU, held until the process ends. Host code never uses the array's
// name as an address (on the host it is only a stand-in for the symbol);
// every use goes through the device address fetched per device below.
constexpr int64_t kNoAllocScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

void* g_scratch_ptr[kMaxDev];
std::mutex g_scratch_mu;

// this device's address of `scratch` (fetched once, with the device current)
svdq_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return fail(SVDQ_ERR_DEVICE, "no current HIP device");
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(SVDQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SVDQ_OK;
}

}  // namespace

svdq_status svdq_gemm_w4a4_quant_next_noalloc(const uint8_t* qx, const void* sx_f16, int64_t M, int64_t K,
                                              const uint8_t* qw, const void* sw_f16, int64_t N,
                                              const float* xl1, const void* l2t, int32_t rank,
                                              const void* bias, int32_t act,
                                              const float* inv_lambda_next, const void* l1t_next, int32_t rank_next,
                                              uint8_t* qx_next, void* sx_next_f16, float* xl1_next, void* stream) {
    svdq_status s;
    if ((s = check_next_shape(M, N, rank_next)) != SVDQ_OK) return s;
    const int64_t need = gemm_next_partial_bytes(M, N, rank_next);
    if (need > kNoAllocScratchBytes)
        return fail(SVDQ_ERR_SHAPE, "the tile partials take %lld bytes, above the %lld bytes of the built-in scratch "
                    "(use svdq_gemm_w4a4_quant_next with a workspace)", (long long)need,
                    (long long)kNoAllocScratchBytes);
    void* ws = nullptr;
    if (rank_next > 0 && M > 0) {
        if ((s = check_current_device()) != SVDQ_OK) return s;
        if ((s = scratch_address(&ws)) != SVDQ_OK) return s;
    }
    return svdq_gemm_w4a4_quant_next(qx, sx_f16, M, K, qw, sw_f16, N, xl1, l2t, rank, bias, act, inv_lambda_next,
                                     l1t_next, rank_next, qx_next, sx_next_f16, xl1_next, ws, need, stream);
}
