// Offline quantiser on the GPU: what turns a bf16 weight into an SVDQ layer
// (donmalab.com page, section on quantising a model yourself: the Quantize
// step produces the 4-bit weights and the low-rank branch; remio.ai page,
// section on SVDQuant moving hard values out of 4-bit: calibration statistics
// shape the smoothing, the low-rank branch takes the hardest part of the
// smoothed weight, the residual is quantised to 4 bits).
//
// Steps, each a kernel (or a short sequence) on the caller's stream:
//  - calibration maxima: ax[k] = max_m |X[m,k]| over a calibration batch
//    (optionally folded into the maxima of earlier batches), aw[k] =
//    max_n |W[k,n]|;
//  - smoothing: lambda = ax^alpha / aw^(1-alpha) in fp64 (1 where either
//    maximum is 0), stored as inv_lambda = fp32(1 / lambda);
//  - smoothed weight: W_hat[k,n] = W[k,n] / inv_lambda[k] in fp64, so that
//    the online path's x * inv_lambda times W_hat is X W in real arithmetic;
//  - truncated SVD of W_hat by the randomised range finder with power
//    iterations (Halko, Martinsson and Tropp, SIAM Review 2011, algorithms
//    4.3/4.4 and 5.1): Y = W_hat Omega, orthonormalise, then alternately
//    through W_hat^T and W_hat; the l x N projection B = Q^T W_hat is
//    decomposed through the eigenvectors of B B^T (cyclic Jacobi).
//    L1 = bf16(U_r Sigma_r), L2 = bf16(V_r^T), each rounded once from fp64,
//    with the largest-magnitude entry of every right singular vector made
//    positive. The random test matrix Omega is an input;
//  - residual R = W_hat - L1 L2 (fp64 from the rounded factors, then fp32),
//    symmetric INT4 per (column, group of 64 along K) with fp16 scales,
//    written straight in the layouts the GEMM reads (codes format v2,
//    scales format v3);
//  - the factors in the layouts the online kernels read (L1 tiles format
//    v4, L2 transposed to [N][r]).
//
// CDNA4 mapping: the maxima and the residual pass are HBM streams (one
// thread per column and group for the residual, W_hat read once, coalesced
// along N). The range finder's products are tall-skinny fp64 GEMMs (N or K
// long, l <= 88 wide), LDS-tiled on the fp64 VALU and split along their long
// dimension so that about 512 workgroups stream W_hat; split partials are
// summed in a fixed order, so every result is deterministic. The l x l work
// (Cholesky, triangular inverse, Jacobi) runs in one workgroup out of LDS.
// Orthonormalisation is CholeskyQR applied twice: the Gram matrix of the
// block, its Cholesky factor R, the block times R^-1 (a column whose pivot
// vanishes, i.e. lies in the span of the earlier ones, becomes zero).
#include "common.h"
#include "int4_fields.h"

namespace {

// ---------------------------------------------------------------------------
// calibration maxima

// axis 0: out[c] = max_r |a[r][c]|. Each lane owns 8 consecutive columns (one
// 16-byte load per row); the rows are split over the grid's y dimension and
// the partial maxima meet in `out` through an atomic max on the bit pattern
// (non-negative floats order like their bits), so the result does not
// depend on the order.
__global__ __launch_bounds__(256) void absmax_cols_kernel(const uint16_t* __restrict__ a, int64_t rows,
                                                          int64_t cols, int64_t lda, int64_t rows_per,
                                                          uint32_t* __restrict__ out) {
    const int64_t c8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c8 >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per;
    const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t r = r0; r < r1; ++r) {
        const uint4 v = *(const uint4*)(a + r * lda + c8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m[2 * j] = fmaxf(m[2 * j], fabsf(bf16_lo_to_f32(w[j])));
            m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16_hi_to_f32(w[j])));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) atomicMax(out + c8 + j, __float_as_uint(m[j]));
}

// axis 1: out[r] = max_c |a[r][c]|, one wave per row.
__global__ __launch_bounds__(256) void absmax_rows_kernel(const uint16_t* __restrict__ a, int64_t rows,
                                                          int64_t cols, int64_t lda, uint32_t* __restrict__ out) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    float m = 0.f;
    for (int64_t c8 = (int64_t)lane * 8; c8 < cols; c8 += 512) {
        const uint4 v = *(const uint4*)(a + r * lda + c8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m = fmaxf(m, fmaxf(fabsf(bf16_lo_to_f32(w[j])), fabsf(bf16_hi_to_f32(w[j]))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) atomicMax(out + r, __float_as_uint(m));
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// smoothing

__global__ void smoothing_kernel(const float* __restrict__ ax, const float* __restrict__ aw, int64_t K,
                                 double alpha, float* __restrict__ inv_lambda) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    const double x = ax[k], w = aw[k];
    double lam = 1.0;
    if (x > 0.0 && w > 0.0) {
        // x^0.5 and w^0.5 are square roots (correctly rounded); other
        // exponents go through pow
        lam = alpha == 0.5 ? sqrt(x) / sqrt(w) : pow(x, alpha) / pow(w, 1.0 - alpha);
    }
    inv_lambda[k] = (float)(1.0 / lam);
}

// W_hat[k, n] = f64(W[k, n]) / f64(inv_lambda[k]); 8 columns per thread
__global__ __launch_bounds__(256) void smooth_weight_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                            int64_t N, int64_t ldw,
                                                            const float* __restrict__ inv_lambda,
                                                            double* __restrict__ w_hat) {
    const int64_t n8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    const int64_t k = blockIdx.y;
    if (n8 >= N) return;
    const double d = inv_lambda ? (double)inv_lambda[k] : 1.0;
    const uint4 v = *(const uint4*)(w + k * ldw + n8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    double o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = (double)bf16_lo_to_f32(u[j]) / d;
        o[2 * j + 1] = (double)bf16_hi_to_f32(u[j]) / d;
    }
    double* dst = w_hat + k * N + n8;
#pragma unroll
    for (int j = 0; j < 8; j += 2) *(double2*)(dst + j) = make_double2(o[j], o[j + 1]);
}

// ---------------------------------------------------------------------------
// tall-skinny fp64 products

// P_s = op(A)[i0:i0+64, ks:ke] * B[ks:ke, 0:nc] for the split s = blockIdx.y
// (op(A) = A, or A^T when TA). op(A) is M x Kd; B is Kd x nc with nc <= 128;
// the result goes to C (one split) or to the partial buffer P[s][M][nc].
// Each of the 256 threads owns 4 rows x 8 columns (cols c, c + 16, ...).
template <bool TA>
__global__ __launch_bounds__(256) void gemm_f64_kernel(const double* __restrict__ A, int64_t lda,
                                                       const double* __restrict__ B, int64_t ldb,
                                                       double* __restrict__ C, int64_t ldc, int64_t M, int nc,
                                                       int64_t Kd, int64_t kchunk) {
    __shared__ double As[16][65];
    __shared__ double Bs[16][128];
    const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
    const int64_t i0 = (int64_t)blockIdx.x * 64;
    const int64_t ks = (int64_t)blockIdx.y * kchunk;
    const int64_t ke = ks + kchunk < Kd ? ks + kchunk : Kd;
    double acc[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] = 0.0;
    for (int64_t k0 = ks; k0 < ke; k0 += 16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = t + 256 * e;
            const int ii = TA ? (idx & 63) : (idx >> 4), kk = TA ? (idx >> 6) : (idx & 15);
            const int64_t i = i0 + ii, k = k0 + kk;
            As[kk][ii] = (i < M && k < ke) ? (TA ? A[k * lda + i] : A[i * lda + k]) : 0.0;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = t + 256 * e;
            const int kk = idx >> 7, c = idx & 127;
            const int64_t k = k0 + kk;
            Bs[kk][c] = (k < ke && c < nc) ? B[k * ldb + c] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            double a[4], b[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = As[kk][rg * 4 + r];
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = Bs[kk][cg + 16 * j];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[r][j] = fma(a[r], b[j], acc[r][j]);
        }
        __syncthreads();
    }
    double* dst = C + (int64_t)blockIdx.y * M * ldc;     // split s writes its own slab
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t i = i0 + rg * 4 + r;
        if (i >= M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = cg + 16 * j;
            if (c < nc) dst[i * ldc + c] = acc[r][j];
        }
    }
}

// C[i][c] = sum over s in order of P[s][i][c]
__global__ void sum_splits_kernel(const double* __restrict__ P, int S, int64_t M, int nc,
                                  double* __restrict__ C, int64_t ldc) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= M * nc) return;
    const int64_t i = e / nc;
    const int c = (int)(e - i * nc);
    double v = 0.0;
    for (int s = 0; s < S; ++s) v += P[(int64_t)s * M * nc + e];
    C[i * ldc + c] = v;
}

// ---------------------------------------------------------------------------
// l x l work in one workgroup

constexpr int LMAX = 88;          // block width the small kernels hold in LDS (2 x 88^2 doubles)

// Rinv = R^-1 for the Cholesky factor R of the Gram matrix G = R^T R (upper
// triangular). A pivot that is not above eps^2 of its diagonal entry marks a
// column that lies in the span of the earlier ones: its row of R is set to
// e_j and its column of Rinv to zero, so the orthonormalised block gets a
// zero column there.
__global__ __launch_bounds__(256) void chol_inv_kernel(const double* __restrict__ G, int l,
                                                       double* __restrict__ Rinv) {
    __shared__ double R[LMAX][LMAX + 1];
    __shared__ int dead[LMAX];
    __shared__ double piv;
    const int t = threadIdx.x;
    for (int e = t; e < l * l; e += 256) R[e / l][e % l] = G[e];
    __syncthreads();
    for (int j = 0; j < l; ++j) {
        if (t == 0) {
            const double d = R[j][j];
            const double ref = G[j * l + j];
            const bool ok = d > 1e-28 * ref && d > 0.0;
            dead[j] = ok ? 0 : 1;
            piv = ok ? sqrt(d) : 1.0;
        }
        __syncthreads();
        const int dj = dead[j];
        const double p = piv;
        for (int c = j + 1 + t; c < l; c += 256) R[j][c] = dj ? 0.0 : R[j][c] / p;
        if (t == 0) R[j][j] = p;
        __syncthreads();
        // trailing update of the upper triangle: R[a][c] -= R[j][a] R[j][c]
        const int n = l - j - 1;
        for (int e = t; e < n * n; e += 256) {
            const int a = j + 1 + e / n, c = j + 1 + e % n;
            if (c >= a) R[a][c] -= R[j][a] * R[j][c];
        }
        __syncthreads();
    }
    // column c of Rinv by back substitution (thread c); dead columns are zero
    for (int c = t; c < l; c += 256) {
        for (int i = l - 1; i >= 0; --i) {
            double v;
            if (i > c) v = 0.0;
            else if (i == c) v = dead[c] ? 0.0 : 1.0 / R[c][c];
            else {
                double s = 0.0;
                for (int m = i + 1; m <= c; ++m) s = fma(R[i][m], Rinv[m * l + c], s);
                v = -s / R[i][i];
            }
            Rinv[i * l + c] = v;
        }
    }
}

// Eigen-decomposition of the symmetric l x l matrix G by cyclic Jacobi in the
// round-robin order (all l/2 disjoint rotations of a round at once), until
// the off-diagonal mass is below 1e-30 of the total or 60 sweeps have run.
// ev gets the eigenvalues in descending order, V (row-major) the matching
// eigenvectors as columns.
constexpr int LS = LMAX + 1;      // row stride of the l x l matrices in LDS
constexpr size_t kEigLds = (size_t)2 * LMAX * LS * sizeof(double);

__global__ __launch_bounds__(256) void sym_eig_kernel(const double* __restrict__ G, int l,
                                                      double* __restrict__ ev, double* __restrict__ V) {
    extern __shared__ double eig_smem[];
    double (*A)[LS] = (double (*)[LS])eig_smem;                 // the matrix being diagonalised
    double (*Q)[LS] = (double (*)[LS])(eig_smem + LMAX * LS);   // accumulated rotations
    __shared__ double cs[LMAX / 2][2];
    __shared__ int pr[LMAX / 2][2];
    __shared__ int order[LMAX];
    __shared__ double red[256];
    __shared__ int done;
    const int t = threadIdx.x;
    const int lp = l + (l & 1);                       // a zero row and column pad an odd size
    for (int e = t; e < lp * lp; e += 256) {
        const int i = e / lp, j = e % lp;
        A[i][j] = (i < l && j < l) ? G[i * l + j] : 0.0;
        Q[i][j] = i == j ? 1.0 : 0.0;
    }
    __syncthreads();
    const int half = lp / 2;
    for (int sweep = 0; sweep < 60; ++sweep) {
        // convergence: off-diagonal against total mass
        double off = 0.0, tot = 0.0;
        for (int e = t; e < lp * lp; e += 256) {
            const int i = e / lp, j = e % lp;
            const double v = A[i][j] * A[i][j];
            tot += v;
            if (i != j) off += v;
        }
        red[t] = off;
        __syncthreads();
        if (t == 0) {
            double o = 0.0;
            for (int i = 0; i < 256; ++i) o += red[i];
            red[0] = o;
        }
        __syncthreads();
        const double offs = red[0];
        __syncthreads();
        red[t] = tot;
        __syncthreads();
        if (t == 0) {
            double s = 0.0;
            for (int i = 0; i < 256; ++i) s += red[i];
            done = !(offs > 1e-30 * s);
        }
        __syncthreads();
        if (done) break;
        for (int round = 0; round < lp - 1; ++round) {
            // pairs of this round: player 0 fixed, the others rotate
            for (int q = t; q < half; q += 256) {
                auto player = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + round) % (lp - 1); };
                int p0 = player(q), p1 = player(lp - 1 - q);
                if (p0 > p1) { const int x = p0; p0 = p1; p1 = x; }
                pr[q][0] = p0;
                pr[q][1] = p1;
                const double apq = A[p0][p1];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    const double theta = (A[p1][p1] - A[p0][p0]) / (2.0 * apq);
                    const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
                    c = 1.0 / sqrt(1.0 + tt * tt);
                    s = tt * c;
                }
                cs[q][0] = c;
                cs[q][1] = s;
            }
            __syncthreads();
            // rows p, q of A (A <- J^T A)
            for (int e = t; e < half * lp; e += 256) {
                const int q = e / lp, m = e % lp;
                const int p0 = pr[q][0], p1 = pr[q][1];
                const double c = cs[q][0], s = cs[q][1];
                const double x = A[p0][m], y = A[p1][m];
                A[p0][m] = c * x - s * y;
                A[p1][m] = s * x + c * y;
            }
            __syncthreads();
            // columns p, q of A (A <- A J) and of the eigenvector matrix
            for (int e = t; e < half * lp; e += 256) {
                const int q = e / lp, m = e % lp;
                const int p0 = pr[q][0], p1 = pr[q][1];
                const double c = cs[q][0], s = cs[q][1];
                const double x = A[m][p0], y = A[m][p1];
                A[m][p0] = c * x - s * y;
                A[m][p1] = s * x + c * y;
                const double u = Q[m][p0], v = Q[m][p1];
                Q[m][p0] = c * u - s * v;
                Q[m][p1] = s * u + c * v;
            }
            __syncthreads();
        }
    }
    // descending order, stable in the index
    if (t == 0) {
        for (int i = 0; i < l; ++i) order[i] = i;
        for (int i = 0; i < l; ++i) {
            int best = i;
            for (int j = i + 1; j < l; ++j)
                if (A[order[j]][order[j]] > A[order[best]][order[best]]) best = j;
            const int x = order[i];
            order[i] = order[best];
            order[best] = x;
        }
    }
    __syncthreads();
    for (int e = t; e < l * l; e += 256) {
        const int i = e / l, j = e % l;
        V[i * l + j] = Q[i][order[j]];
    }
    for (int j = t; j < l; j += 256) ev[j] = A[order[j]][order[j]];
}

// sign of each right singular vector: the entry of largest magnitude (first
// index among equals) is made positive. One workgroup per vector i of the
// unnormalised V (N x ldv, column i).
__global__ __launch_bounds__(256) void sign_kernel(const double* __restrict__ V, int64_t N, int ldv,
                                                   double* __restrict__ sgn) {
    __shared__ double bv[256];
    __shared__ int64_t bi[256];
    const int i = blockIdx.x, t = threadIdx.x;
    double best = -1.0;
    int64_t at = 0;
    for (int64_t n = t; n < N; n += 256) {
        const double a = fabs(V[n * ldv + i]);
        if (a > best) { best = a; at = n; }
    }
    bv[t] = best;
    bi[t] = at;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (t < o) {
            const double b2 = bv[t + o];
            const int64_t i2 = bi[t + o];
            if (b2 > bv[t] || (b2 == bv[t] && i2 < bi[t])) { bv[t] = b2; bi[t] = i2; }
        }
        __syncthreads();
    }
    if (t == 0) sgn[i] = V[bi[0] * ldv + i] < 0.0 ? -1.0 : 1.0;
}

// fp64 -> bf16 bits with one round to nearest even: truncate to fp32, make
// the last fp32 bit sticky when anything was cut off (round to odd), then
// let the native conversion round that to bf16. fp32 keeps 16 more bits
// than bf16, so the sticky bit decides ties exactly as the fp64 value would.
DEV uint16_t f64_to_bf16_bits(double x) {
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
    return f32_to_bf16_bits(f);
}

// L1[k][i] = bf16(sgn_i sigma_i U[k][i]), U = Q U_B (K x r, leading dim ldu)
__global__ void l1_out_kernel(const double* __restrict__ U, int ldu, int64_t K, int r,
                              const double* __restrict__ ev, const double* __restrict__ sgn,
                              uint16_t* __restrict__ l1) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= K * r) return;
    const int64_t k = e / r;
    const int i = (int)(e - k * r);
    const double sig = sqrt(ev[i] > 0.0 ? ev[i] : 0.0);
    l1[e] = f64_to_bf16_bits(sgn[i] * (U[k * ldu + i] * sig));
}

// L2[i][n] = bf16(sgn_i V[n][i] / sigma_i) (0 where sigma_i = 0); sigma out
__global__ void l2_out_kernel(const double* __restrict__ V, int ldv, int64_t N, int r,
                              const double* __restrict__ ev, const double* __restrict__ sgn,
                              uint16_t* __restrict__ l2, double* __restrict__ sigma) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= N * r) return;
    const int i = (int)(e / N);
    const int64_t n = e - (int64_t)i * N;
    const double sig = sqrt(ev[i] > 0.0 ? ev[i] : 0.0);
    l2[e] = sig > 0.0 ? f64_to_bf16_bits(sgn[i] * (V[n * ldv + i] / sig)) : (uint16_t)0;
    if (sigma && n == 0) sigma[i] = sig;
}

// ---------------------------------------------------------------------------
// residual quantisation

// One thread per (column n, group g): R[k][n] = fp32(W_hat[k][n] - sum_j
// L1[k][j] L2[j][n]) for the 64 k of the group (the products of two bf16
// values are exact in fp64), then the symmetric INT4 quantisation with the
// stored fp16 scale: s = fp16(min(amax / 7, 65504)), inv = fp32(1 / s),
// q = clamp(rtne(R inv), -7, 7), zero codes when s = 0. The 64 codes go out
// as four format-v2 words at qw[n][32 g ..], the scale at its quad-major
// place sw[g / 4][n][g % 4]. The group's L1 rows sit in LDS; the thread's
// column of L2 in registers.
template <int RT>
__global__ __launch_bounds__(256) void residual_q_kernel(const double* __restrict__ w_hat, int64_t K, int64_t N,
                                                         const uint16_t* __restrict__ l1,
                                                         const uint16_t* __restrict__ l2,
                                                         uint8_t* __restrict__ qw, uint16_t* __restrict__ sw) {
    constexpr int R = RT * 16;
    __shared__ float s_l1[64][R > 0 ? R : 1];
    const int64_t g = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int e = threadIdx.x; e < 64 * R; e += 256) {
        const int kk = e / (R > 0 ? R : 1), j = e % (R > 0 ? R : 1);
        s_l1[kk][j] = __uint_as_float((uint32_t)l1[(g * 64 + kk) * R + j] << 16);
    }
    __syncthreads();
    if (n >= N) return;
    float l2c[R > 0 ? R : 1];
#pragma unroll
    for (int j = 0; j < R; ++j) l2c[j] = __uint_as_float((uint32_t)l2[(int64_t)j * N + n] << 16);
    float v[64];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 64; ++kk) {
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < R; ++j) s = fma((double)s_l1[kk][j], (double)l2c[j], s);
        v[kk] = (float)(w_hat[(g * 64 + kk) * N + n] - s);
        amax = fmaxf(amax, fabsf(v[kk]));
    }
    const float s32 = fminf(amax / 7.0f, 65504.0f);
    const _Float16 s16 = (_Float16)s32;
    const float sf = (float)s16;
    const float inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;
    uint8_t* dst = qw + n * (K / 2) + g * 32;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        uint32_t f[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) f[j] = code_field(v[16 * wd + j], inv);
        *(uint2*)(dst + 8 * wd) = fold_fields(f);
    }
    sw[((g >> 2) * N + n) * 4 + (g & 3)] = __builtin_bit_cast(uint16_t, s16);
}

// The MXFP4 form of the residual quantisation (the number format of the
// MXFP4 layer, OCP Microscaling Formats v1.0): the same residual values of
// one (output column n, group g of 64), then per 32-value block its E8M0
// exponent e = floor(log2 amax) - 2 (clamped; -127 for a zero block) and the
// E2M1 codes of R * 2^-e, rounded to nearest with ties to mantissa 0 and
// saturating at 6, a zero with sign 0 (the activation kernel's MXFP4 step).
// The 64 nibbles go to qw[n][32 g ..] (element 2i in bits 0-3 of byte i),
// the two exponent bytes (e + 127) to the group's places in the records
// [ceil(G/4)][N][8]: block 2 (g % 4) at byte g % 4, block 2 (g % 4) + 1 at
// byte 4 + g % 4.
template <int RT>
__global__ __launch_bounds__(256) void residual_mx_kernel(const double* __restrict__ w_hat, int64_t K, int64_t N,
                                                          const uint16_t* __restrict__ l1,
                                                          const uint16_t* __restrict__ l2,
                                                          uint8_t* __restrict__ qw, uint8_t* __restrict__ se) {
    constexpr int R = RT * 16;
    __shared__ float s_l1[64][R > 0 ? R : 1];
    const int64_t g = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int e = threadIdx.x; e < 64 * R; e += 256) {
        const int kk = e / (R > 0 ? R : 1), j = e % (R > 0 ? R : 1);
        s_l1[kk][j] = __uint_as_float((uint32_t)l1[(g * 64 + kk) * R + j] << 16);
    }
    __syncthreads();
    if (n >= N) return;
    float l2c[R > 0 ? R : 1];
#pragma unroll
    for (int j = 0; j < R; ++j) l2c[j] = __uint_as_float((uint32_t)l2[(int64_t)j * N + n] << 16);
    uint8_t* dst = qw + n * (K / 2) + g * 32;
    uint8_t* rec = se + ((g >> 2) * N + n) * 8 + (g & 3);
    for (int b = 0; b < 2; ++b) {
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) {
            const int64_t k = g * 64 + 32 * b + kk;
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < R; ++j) s = fma((double)s_l1[32 * b + kk][j], (double)l2c[j], s);
            v[kk] = (float)(w_hat[k * N + n] - s);
            amax = fmaxf(amax, fabsf(v[kk]));
        }
        const int e = mx_block_exponent(amax);
        const float sc = mx_inv_scale(e);
        float t[32];
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) t[kk] = v[kk] * sc;
        *(uint4*)(dst + 16 * b) = make_uint4(e2m1_x8(t), e2m1_x8(t + 8), e2m1_x8(t + 16), e2m1_x8(t + 24));
        rec[4 * b] = (uint8_t)(e + 127);
    }
}

// groups past the last one in the quad-major scale array hold 0
__global__ void sw_pad_kernel(uint16_t* __restrict__ sw, int64_t N, int G) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    for (int g = G; g < ((G + 3) & ~3); ++g) sw[((int64_t)(g >> 2) * N + n) * 4 + (g & 3)] = 0;
}

// ---------------------------------------------------------------------------
// factor layouts of the online kernels

// L1 tiles (format v4): for group g, 16-rank tile t, step s, lane l: the 8
// values L1[64 g + 16 (l / 16) + 8 s + j][16 t + l % 16], j = 0..7
__global__ void pack_l1_kernel(const uint16_t* __restrict__ l1, int64_t K, int r, uint16_t* __restrict__ l1t) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;     // one thread per 8 values
    const int T = r / 16;
    if (e >= K / 64 * T * 128) return;
    const int lane = (int)(e & 63), st = (int)((e >> 6) & 1);
    const int64_t gt = e >> 7;
    const int t = (int)(gt % T);
    const int64_t g = gt / T;
    const int64_t k0 = 64 * g + 16 * (lane >> 4) + 8 * st;
    const int col = 16 * t + (lane & 15);
    uint16_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = l1[(k0 + j) * r + col];
    *(uint4*)(l1t + e * 8) = make_uint4(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16),
                                        o[4] | ((uint32_t)o[5] << 16), o[6] | ((uint32_t)o[7] << 16));
}

// l2t[n][i] = L2[i][n]
__global__ void pack_l2_kernel(const uint16_t* __restrict__ l2, int64_t N, int r, uint16_t* __restrict__ l2t) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= N * r) return;
    const int64_t n = e / r;
    const int i = (int)(e - n * r);
    l2t[e] = l2[(int64_t)i * N + n];
}

int blocks_for(int64_t n, int per) { return (int)((n + per - 1) / per); }

}  // namespace

// ---------------------------------------------------------------------------
// host side (launch sequences; arguments validated by the C ABI layer)

hipError_t launch_calib_absmax(const uint16_t* a, int64_t rows, int64_t cols, int64_t lda, int axis,
                               int accumulate, float* out, hipStream_t stream) {
    uint32_t* o = (uint32_t*)out;
    const int64_t n = axis == 0 ? cols : rows;
    if (!accumulate) hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, stream, o, n, 0u);
    if (rows == 0 || cols == 0) return hipGetLastError();
    if (axis == 0) {
        const int cb = blocks_for(cols, 256 * 8);
        int64_t split = 1024 / cb;
        if (split < 1) split = 1;
        if (split > rows) split = rows;
        const int64_t per = (rows + split - 1) / split;
        hipLaunchKernelGGL(absmax_cols_kernel, dim3(cb, (unsigned)((rows + per - 1) / per)), dim3(256), 0, stream,
                           a, rows, cols, lda, per, o);
    } else {
        hipLaunchKernelGGL(absmax_rows_kernel, dim3(blocks_for(rows, 4)), dim3(256), 0, stream, a, rows, cols, lda, o);
    }
    return hipGetLastError();
}

hipError_t launch_smoothing(const float* ax, const float* aw, int64_t K, double alpha, float* inv_lambda,
                            hipStream_t stream) {
    hipLaunchKernelGGL(smoothing_kernel, dim3(blocks_for(K, 256)), dim3(256), 0, stream, ax, aw, K, alpha, inv_lambda);
    return hipGetLastError();
}

hipError_t launch_smooth_weight(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, const float* inv_lambda,
                                double* w_hat, hipStream_t stream) {
    hipLaunchKernelGGL(smooth_weight_kernel, dim3(blocks_for(N, 256 * 8), (unsigned)K), dim3(256), 0, stream,
                       w, K, N, ldw, inv_lambda, w_hat);
    return hipGetLastError();
}

namespace {

// the range finder's scratch, carved from the caller's workspace
struct LowrankWs {
    double *y, *z, *t1, *t2, *g, *rinv, *ub, *ev, *sgn, *part;
};

constexpr int64_t kPartDoubles = (int64_t)512 * 64 * 128;   // split partials: <= 512 tiles of 64 x 128

int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

int64_t lowrank_ws_bytes(int64_t K, int64_t N, int l) {
    const int64_t kn = K > N ? K : N;
    return 4 * align256(kn * l * 8) + 3 * align256((int64_t)l * l * 8) + 2 * align256((int64_t)l * 8) +
           align256(kPartDoubles * 8);
}

LowrankWs carve(void* ws, int64_t K, int64_t N, int l) {
    const int64_t kn = K > N ? K : N;
    char* p = (char*)ws;
    LowrankWs w;
    auto take = [&](int64_t bytes) { double* q = (double*)p; p += align256(bytes); return q; };
    w.y = take(kn * l * 8);
    w.z = take(kn * l * 8);
    w.t1 = take(kn * l * 8);
    w.t2 = take(kn * l * 8);
    w.g = take((int64_t)l * l * 8);
    w.rinv = take((int64_t)l * l * 8);
    w.ub = take((int64_t)l * l * 8);
    w.ev = take((int64_t)l * 8);
    w.sgn = take((int64_t)l * 8);
    w.part = take(kPartDoubles * 8);
    return w;
}

// C (M x nc, ldc) = op(A) (M x Kd) * B (Kd x nc, ldb), split along Kd so that
// about 512 workgroups run; the splits are summed in order
template <bool TA>
void gemm_f64(const double* A, int64_t lda, const double* B, int64_t ldb, double* C, int64_t ldc, int64_t M,
              int nc, int64_t Kd, double* part, hipStream_t stream) {
    const int64_t mt = (M + 63) / 64;
    int64_t S = 512 / mt;
    const int64_t smax = Kd / 256 > 0 ? Kd / 256 : 1;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    if (S * mt * 64 * 128 > kPartDoubles) S = 1;
    int64_t kchunk = (Kd + S - 1) / S;
    kchunk = (kchunk + 15) & ~(int64_t)15;
    S = (Kd + kchunk - 1) / kchunk;
    if (S <= 1) {
        hipLaunchKernelGGL(gemm_f64_kernel<TA>, dim3((unsigned)mt, 1), dim3(256), 0, stream, A, lda, B, ldb, C, ldc,
                           M, nc, Kd, Kd > 0 ? Kd : 1);
        return;
    }
    hipLaunchKernelGGL(gemm_f64_kernel<TA>, dim3((unsigned)mt, (unsigned)S), dim3(256), 0, stream, A, lda, B, ldb,
                       part, (int64_t)nc, M, nc, Kd, kchunk);
    hipLaunchKernelGGL(sum_splits_kernel, dim3(blocks_for(M * nc, 256)), dim3(256), 0, stream, part, (int)S, M, nc,
                       C, ldc);
}

// one CholeskyQR pass: dst (rows x l) = src R^-1, R the Cholesky factor of src^T src
void cholqr_pass(const double* src, double* dst, int64_t rows, int l, LowrankWs& w, hipStream_t stream) {
    gemm_f64<true>(src, l, src, l, w.g, l, l, l, rows, w.part, stream);         // G = src^T src
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(256), 0, stream, w.g, l, w.rinv);
    gemm_f64<false>(src, l, w.rinv, l, dst, l, rows, l, l, w.part, stream);     // dst = src R^-1
}

// X (rows x l) orthonormalised in place by CholeskyQR twice (tmp: rows x l)
void orthonormalise(double* X, int64_t rows, int l, double* tmp, LowrankWs& w, hipStream_t stream) {
    cholqr_pass(X, tmp, rows, l, w, stream);
    cholqr_pass(tmp, X, rows, l, w, stream);
}

}  // namespace

int64_t offline_lowrank_ws_bytes(int64_t K, int64_t N, int l) { return lowrank_ws_bytes(K, N, l); }
int offline_lmax() { return LMAX; }

hipError_t launch_lowrank(const double* w_hat, int64_t K, int64_t N, int r, const double* omega, int l,
                          int power_iters, uint16_t* l1, uint16_t* l2, double* sigma, void* ws,
                          hipStream_t stream) {
    LowrankWs w = carve(ws, K, N, l);
    // Q: K x l (in w.y), Z: N x l (in w.z)
    gemm_f64<false>(w_hat, N, omega, l, w.y, l, K, l, N, w.part, stream);        // Y = W_hat Omega
    orthonormalise(w.y, K, l, w.t1, w, stream);
    for (int it = 0; it < power_iters; ++it) {
        gemm_f64<true>(w_hat, N, w.y, l, w.z, l, N, l, K, w.part, stream);       // Z = W_hat^T Q
        orthonormalise(w.z, N, l, w.t2, w, stream);
        gemm_f64<false>(w_hat, N, w.z, l, w.y, l, K, l, N, w.part, stream);      // Y = W_hat Z
        orthonormalise(w.y, K, l, w.t1, w, stream);
    }
    gemm_f64<true>(w_hat, N, w.y, l, w.z, l, N, l, K, w.part, stream);           // B^T = W_hat^T Q
    gemm_f64<true>(w.z, l, w.z, l, w.g, l, l, l, N, w.part, stream);             // B B^T
    (void)hipFuncSetAttribute((const void*)sym_eig_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kEigLds);
    hipLaunchKernelGGL(sym_eig_kernel, dim3(1), dim3(256), kEigLds, stream, w.g, l, w.ev, w.ub);
    gemm_f64<false>(w.y, l, w.ub, l, w.t1, l, K, r, l, w.part, stream);          // U = Q U_B (r columns)
    gemm_f64<false>(w.z, l, w.ub, l, w.t2, l, N, r, l, w.part, stream);          // V sigma = B^T U_B
    hipLaunchKernelGGL(sign_kernel, dim3(r), dim3(256), 0, stream, w.t2, N, l, w.sgn);
    hipLaunchKernelGGL(l1_out_kernel, dim3(blocks_for(K * r, 256)), dim3(256), 0, stream, w.t1, l, K, r, w.ev, w.sgn, l1);
    hipLaunchKernelGGL(l2_out_kernel, dim3(blocks_for(N * r, 256)), dim3(256), 0, stream, w.t2, l, N, r, w.ev, w.sgn,
                       l2, sigma);
    return hipGetLastError();
}

hipError_t launch_quantize_residual(const double* w_hat, int64_t K, int64_t N, const uint16_t* l1,
                                    const uint16_t* l2, int r, uint8_t* qw, uint16_t* sw, hipStream_t stream) {
    const dim3 grid((unsigned)blocks_for(N, 256), (unsigned)(K / 64));
    switch (r / 16) {
        case 0: hipLaunchKernelGGL(residual_q_kernel<0>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 1: hipLaunchKernelGGL(residual_q_kernel<1>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 2: hipLaunchKernelGGL(residual_q_kernel<2>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 3: hipLaunchKernelGGL(residual_q_kernel<3>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 4: hipLaunchKernelGGL(residual_q_kernel<4>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 5: hipLaunchKernelGGL(residual_q_kernel<5>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 6: hipLaunchKernelGGL(residual_q_kernel<6>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        case 7: hipLaunchKernelGGL(residual_q_kernel<7>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, sw); break;
        default: return hipErrorInvalidValue;
    }
    const int G = (int)(K / 64);
    if (G % 4) hipLaunchKernelGGL(sw_pad_kernel, dim3(blocks_for(N, 256)), dim3(256), 0, stream, sw, N, G);
    return hipGetLastError();
}

// AWQ W4A16 weight quantisation (the textbook asymmetric min/max group
// quantiser the GEMV consumes, with the activation-aware channel scale folded
// into the weight): one thread per (output column n, group g of 64 input
// channels). W' = fp32(W / inv_s) (the division in fp64, one rounding); mn,
// mx of the group; s = fp16(max(mx - mn, 1e-5) / 15) in fp32; z =
// clamp(rtne(-mn * fp32(1 / s)), 0, 15) kept as an fp16 integer; q =
// clamp(rtne(W' * fp32(1 / s)) + z, 0, 15). The 32 code bytes of the group go
// to their place in the GEMV tile layout [N/16][K/128][16][64 B] (block
// (t, j, c) = bytes 64 j .. 64 j + 63 of column 16 t + c's packed row, element
// 2i in bits 0-3 of byte i), s and z to [N/16][K/64][16].
__global__ __launch_bounds__(256) void awq_quantize_kernel(const uint16_t* __restrict__ w, int64_t K, int64_t N,
                                                           int64_t ldw, const float* __restrict__ inv_s,
                                                           uint8_t* __restrict__ qwt, uint16_t* __restrict__ sc,
                                                           uint16_t* __restrict__ zr) {
    const int64_t g = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float v[64];
    float mn = 0.0f, mx = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 64; ++kk) {
        const int64_t k = g * 64 + kk;
        const double wv = (double)__uint_as_float((uint32_t)w[k * ldw + n] << 16);
        v[kk] = inv_s ? (float)(wv / (double)inv_s[k]) : (float)wv;
        mn = kk == 0 ? v[kk] : fminf(mn, v[kk]);
        mx = kk == 0 ? v[kk] : fmaxf(mx, v[kk]);
    }
    const float rng = fmaxf(mx - mn, 1e-5f);
    const _Float16 s16 = (_Float16)(rng / 15.0f);
    const float inv = 1.0f / (float)s16;
    const float z = fminf(fmaxf(rintf(-mn * inv), 0.0f), 15.0f);
    uint32_t wd[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = fminf(fmaxf(rintf(v[8 * d + e] * inv) + z, 0.0f), 15.0f);
            word |= (uint32_t)q << (4 * e);
        }
        wd[d] = word;
    }
    const int64_t t = n >> 4, c = n & 15, j = g >> 1;
    uint8_t* dst = qwt + ((t * (K / 128) + j) * 16 + c) * 64 + (g & 1) * 32;
    *(uint4*)dst = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    *(uint4*)(dst + 16) = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    const int64_t o = (t * (K / 64) + g) * 16 + c;
    sc[o] = __builtin_bit_cast(uint16_t, s16);
    zr[o] = __builtin_bit_cast(uint16_t, (_Float16)z);
}

// exponent bytes of groups past the last one hold 0 (as the packers write them)
__global__ void se_pad_kernel(uint8_t* __restrict__ se, int64_t N, int G) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    for (int g = G; g < ((G + 3) & ~3); ++g) {
        uint8_t* rec = se + ((int64_t)(g >> 2) * N + n) * 8 + (g & 3);
        rec[0] = 0;
        rec[4] = 0;
    }
}

hipError_t launch_quantize_residual_mxfp4(const double* w_hat, int64_t K, int64_t N, const uint16_t* l1,
                                          const uint16_t* l2, int r, uint8_t* qw, uint8_t* se, hipStream_t stream) {
    const dim3 grid((unsigned)blocks_for(N, 256), (unsigned)(K / 64));
    switch (r / 16) {
        case 0: hipLaunchKernelGGL(residual_mx_kernel<0>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 1: hipLaunchKernelGGL(residual_mx_kernel<1>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 2: hipLaunchKernelGGL(residual_mx_kernel<2>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 3: hipLaunchKernelGGL(residual_mx_kernel<3>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 4: hipLaunchKernelGGL(residual_mx_kernel<4>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 5: hipLaunchKernelGGL(residual_mx_kernel<5>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 6: hipLaunchKernelGGL(residual_mx_kernel<6>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        case 7: hipLaunchKernelGGL(residual_mx_kernel<7>, grid, dim3(256), 0, stream, w_hat, K, N, l1, l2, qw, se); break;
        default: return hipErrorInvalidValue;
    }
    const int G = (int)(K / 64);
    if (G % 4) hipLaunchKernelGGL(se_pad_kernel, dim3(blocks_for(N, 256)), dim3(256), 0, stream, se, N, G);
    return hipGetLastError();
}

hipError_t launch_awq_quantize(const uint16_t* w, int64_t K, int64_t N, int64_t ldw, const float* inv_s,
                               uint8_t* qwt, uint16_t* sc, uint16_t* zr, hipStream_t stream) {
    hipLaunchKernelGGL(awq_quantize_kernel, dim3((unsigned)blocks_for(N, 256), (unsigned)(K / 64)), dim3(256), 0,
                       stream, w, K, N, ldw, inv_s, qwt, sc, zr);
    return hipGetLastError();
}

hipError_t launch_pack_lowrank(const uint16_t* l1, const uint16_t* l2, int64_t K, int64_t N, int r, uint16_t* l1t,
                               uint16_t* l2t, hipStream_t stream) {
    if (r == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_l1_kernel, dim3(blocks_for(K / 64 * (r / 16) * 128, 256)), dim3(256), 0, stream, l1, K, r,
                       l1t);
    hipLaunchKernelGGL(pack_l2_kernel, dim3(blocks_for(N * r, 256)), dim3(256), 0, stream, l2, N, r, l2t);
    return hipGetLastError();
}
