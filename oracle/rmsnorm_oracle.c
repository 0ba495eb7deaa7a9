/*
 * Oracle: plain, slow, double-precision CPU reference for fused row-wise
 * RMSNorm (forward, residual-add forward, explicit backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library: no headers, helpers, tables or constants.
 *
 * Sources (the method is defined there; all statements below are restated,
 * not quoted):
 *   P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）"
 *        (iqiancheng.github.io), §4.1 (forward definition), §4.2 (forward
 *        kernel: fp32 upcast, masked tail, divide by the true width),
 *        §5.3 (backward derivation), §5.4 (dw as a cross-row sum).
 *   P2 = the trdm.cn write-up of hand-written Triton decode kernels
 *        (www.trdm.cn/news/483216), §2.1 (residual_add followed by rms_norm,
 *        and the planned fused residual + RMSNorm kernel), §3.1 (the decode
 *        projection as a matrix-vector product, computed with split-K).
 *
 * Every loop runs in natural index order; no blocking, no reordering, no
 * parallelism.  Inputs are the exact values of the (already quantised) I/O
 * tensors, passed as doubles.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* h-storage types for the residual forward (matches the I/O dtype). */
#define ORACLE_H_F32 0
#define ORACLE_H_BF16 1
#define ORACLE_H_EXACT 2 /* keep x + res unrounded (used by derivative pins) */

/* Round a double to the nearest bfloat16 value, ties to even.
 * bfloat16 = 1 sign bit, 8 exponent bits (fp32's range), 8 significant bits.
 * Normal values keep 8 significant bits; below 2^-126 the spacing is fixed at
 * 2^-133 (subnormals); magnitudes that round past the largest finite value
 * (2 - 2^-7) * 2^127 become infinity. */
double oracle_round_bf16(double v) {
    if (!isfinite(v) || v == 0.0) return v;
    int e;
    frexp(v, &e);          /* |v| = m * 2^e with 0.5 <= m < 1: top bit weight 2^(e-1) */
    int q = e - 8;         /* weight of the lowest kept bit */
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(v, -q)), q); /* nearbyint: ties to even */
    const double bf16_max = ldexp(255.0, 120);     /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max) return copysign(INFINITY, v);
    return r;
}

/* Round a double to the nearest fp32 value (C conversion, ties to even). */
double oracle_round_f32(double v) { return (double)(float)v; }

/* rstd of one row: 1 / sqrt(mean of squares + eps), mean over the true width
 * H (P1 §4.1 definition; P1 §4.2 divides the sum by the real width, masked
 * tail lanes contribute zero). */
static double row_rstd(const double *xr, int64_t H, double eps) {
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) ss += xr[j] * xr[j];
    return 1.0 / sqrt(ss / (double)H + eps);
}

/* Forward: y[i][j] = w[j] * x[i][j] * r_i, r_i = 1/sqrt(mean_j x[i][j]^2 + eps)
 * (P1 §4.1).  x, y: [rows][H] row-major; w: [H]; rstd: [rows] (may be NULL). */
void oracle_rmsnorm_fwd(const double *x, const double *w, int64_t rows, int64_t H,
                        double eps, double *y, double *rstd) {
    for (int64_t i = 0; i < rows; ++i) {
        const double *xr = x + i * H;
        double r = row_rstd(xr, H, eps);
        if (rstd) rstd[i] = r;
        for (int64_t j = 0; j < H; ++j) y[i * H + j] = w[j] * xr[j] * r;
    }
}

/* Residual-add + RMSNorm forward (P2 §2.1: residual_add then rms_norm, and
 * the planned fusion of the two):
 *   h = store_T(x + res)       the residual stream, written out in dtype T
 *   y = RMSNorm(h; w, eps)     normalised from the stored h
 * h_kind selects T's rounding: ORACLE_H_F32, ORACLE_H_BF16 or ORACLE_H_EXACT. */
void oracle_rmsnorm_residual_fwd(const double *x, const double *res, const double *w,
                                 int64_t rows, int64_t H, double eps, int h_kind,
                                 double *h, double *y, double *rstd) {
    for (int64_t k = 0; k < rows * H; ++k) {
        double s = x[k] + res[k];
        if (h_kind == ORACLE_H_F32) s = oracle_round_f32(s);
        else if (h_kind == ORACLE_H_BF16) s = oracle_round_bf16(s);
        h[k] = s;
    }
    oracle_rmsnorm_fwd(h, w, rows, H, eps, y, rstd);
}

/* Backward (P1 §5.3):
 *   wdy_j = w_j * dy_j
 *   c     = (1/H) * sum_j wdy_j * x_j                 (per row)
 *   dx_j  = r * (wdy_j - x_j * r^2 * c)   [+ dres_j]
 *   dw_j  = sum over rows of dy_j * x_j * r          (P1 §5.3-§5.4)
 * r is taken from rstd[i] when rstd != NULL (the statistic saved by the
 * forward), otherwise recomputed from x.  dres (nullable) is the gradient of
 * the residual stream arriving from above; with the residual forward, x is h
 * and dx is the gradient of both x and res (h = x + res).
 * dy, x, dx, dres: [rows][H]; w, dw: [H]. */
void oracle_rmsnorm_bwd(const double *dy, const double *x, const double *w,
                        const double *rstd, const double *dres, int64_t rows,
                        int64_t H, double eps, double *dx, double *dw) {
    for (int64_t j = 0; j < H; ++j) dw[j] = 0.0;
    for (int64_t i = 0; i < rows; ++i) {
        const double *xr = x + i * H;
        const double *dyr = dy + i * H;
        double r = rstd ? rstd[i] : row_rstd(xr, H, eps);
        double c = 0.0;
        for (int64_t j = 0; j < H; ++j) c += w[j] * dyr[j] * xr[j];
        c /= (double)H;
        for (int64_t j = 0; j < H; ++j) {
            double g = r * (w[j] * dyr[j] - xr[j] * r * r * c);
            if (dres) g += dres[i * H + j];
            dx[i * H + j] = g;
            dw[j] += dyr[j] * xr[j] * r;
        }
    }
}

/* Decode projection (P2 §3.1): y[n] = sum_k A[n][k] * x[k], A row-major
 * [N][K], x [K], y [N].  Splitting K into segments (the split-K scheme) only
 * regroups this sum; the definition is the plain dot product per row. */
void oracle_gemv(const double *A, const double *x, int64_t N, int64_t K, double *y) {
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += A[n * K + k] * x[k];
        y[n] = s;
    }
}
