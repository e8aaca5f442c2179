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
                            uint8_t* qx, uint16_t* sx, float* xl1, hipStream_t stream);
size_t act_quant_smem_bytes(int64_t K, int rank);
hipError_t launch_gemm_w4a4(const uint8_t* qx, const uint16_t* sx, const uint8_t* qw,
                            const uint16_t* sw, const float* xl1, const uint16_t* l2t, int rank,
                            const uint16_t* bias, int act, void* y, int y_f32, int64_t ldy,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_act_quant_mxfp4(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  const float* inv_lambda, const uint16_t* l1t, int rank,
                                  uint8_t* qx, uint8_t* sx, float* xl1, hipStream_t stream);
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
    if (act_quant_smem_bytes(K, rank) > kMaxLds)
        return fail(SVDQ_ERR_SHAPE, "K = %lld with rank %d exceeds the LDS budget", (long long)K, rank);
    if (M == 0) { g_last_error.clear(); return SVDQ_OK; }   // empty batch: nothing to read or write
    if (!x || !qx || !sx_f16) return fail(SVDQ_ERR_NULL, "x, qx and sx_f16 are required");
    if (rank > 0 && (!l1t || !xl1)) return fail(SVDQ_ERR_NULL, "rank %d needs l1t and xl1", rank);
    if (!aligned(x, 16) || !aligned(qx, 16) || !aligned(sx_f16, 16) ||
        (inv_lambda && !aligned(inv_lambda, 16)) ||
        (rank > 0 && (!aligned(l1t, 16) || !aligned(xl1, 16))))
        return fail(SVDQ_ERR_ALIGN, "x, inv_lambda, l1t, qx, sx_f16, xl1 need 16-byte alignment");
    if ((s = check_current_device()) != SVDQ_OK) return s;
    const uint16_t* l1 = rank > 0 ? (const uint16_t*)l1t : nullptr;
    float* xo = rank > 0 ? xl1 : nullptr;
    if (mxfp4)
        return launched(launch_act_quant_mxfp4((const uint16_t*)x, M, K, ldx, inv_lambda, l1, rank, qx,
                                               (uint8_t*)sx_f16, xo, (hipStream_t)stream),
                        "svdq_quantize_act_mxfp4 launch");
    return launched(launch_act_quant((const uint16_t*)x, M, K, ldx, inv_lambda, l1, rank, qx,
                                     (uint16_t*)sx_f16, xo, (hipStream_t)stream),
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
    if (N <= 0 || N % 8) return fail(SVDQ_ERR_SHAPE, "N = %lld must be a positive multiple of 8", (long long)N);
    if (M > ((int64_t)1 << 31) || N > ((int64_t)1 << 31)) return fail(SVDQ_ERR_SHAPE, "M or N too large");
    if ((s = check_gemm_bytes(M, N, K)) != SVDQ_OK) return s;
    if ((M + 256) * rank * 4 >= ((int64_t)1 << 31) || (N + 256) * rank * 2 >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "(M + 256) * rank * 4 and (N + 256) * rank * 2 must stay below 2^31 bytes");
    if (ldy < N) return fail(SVDQ_ERR_SHAPE, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
    if (ldy % 8) return fail(SVDQ_ERR_ALIGN, "ldy = %lld must be a multiple of 8", (long long)ldy);
    if ((M + 128) * ldy * (y_dtype == SVDQ_DT_F32 ? 4 : 2) >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_SHAPE, "(M + 128) * ldy * element size must stay below 2^31 bytes");
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_UNSUPPORTED, "activation %d is not supported", act);
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

}  // namespace

extern "C" {

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

int svdq_version(void) { return 401; }

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

}  // extern "C"
