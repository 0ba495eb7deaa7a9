// Per-row backward arithmetic shared by the backward row kernels (the
// register-tile, LDS-staged and streaming forms), and their cache hints.
//
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）":
//   §5.3 wdy = w*dy, c = (1/H) sum_j wdy_j x_j, dx = r (wdy - x r^2 c),
//   dw_j = sum over rows of dy_j x_j r.
#pragma once

#include "common.hpp"

// Streaming (nontemporal) access to the row tensors: dy/x/dres loads and
// dx stores (measured best for a forward + backward step: dx lines left
// dirty in the caches are otherwise written back during the next kernel).
#ifndef RMS_BWD_NT_LOAD
#define RMS_BWD_NT_LOAD 1
#endif
#ifndef RMS_BWD_NT_STORE
#define RMS_BWD_NT_STORE 1
#endif
#ifndef RMS_DRES_NT_LOAD
#define RMS_DRES_NT_LOAD 1
#endif
#ifndef RMS_DRES_NT_STORE
#define RMS_DRES_NT_STORE 1
#endif
namespace rms {

// Per-row factors of dx (P1 §5.3): r, k = r^2 c, and k split into two floats
// for the fp32 form.  rf is the dw scale: zero for rows past the end, so
// neither the r of their zero inputs (infinite at eps = 0) nor whatever
// their rstd lane read can turn the 0 * r products into NaN.
struct RowK {
    double r, kk;
    float rf, k_hi, k_lo;
};

__device__ __forceinline__ RowK row_k(double r, double cs, double inv_h, bool active) {
    RowK q;
    q.r = r;
    q.rf = active ? (float)r : 0.f;
    q.kk = r * r * (cs * inv_h);
    q.k_hi = (float)q.kk;
    q.k_lo = (float)(q.kk - (double)q.k_hi);
    return q;
}

// dx of one chunk, dx = r (w dy - x k) [+ dres] (P1 §5.3), and its dw terms
// dy x r added to acc (P1 §5.4; lanes outside the tensor hold zeros and add
// nothing).
template <typename T, int VEC, bool DRES>
__device__ __forceinline__ void dx_chunk(const float (&xv)[VEC], const float (&dyv)[VEC],
                                         const float (&wc)[VEC], const float (&drv)[VEC],
                                         const RowK& q, float (&o)[VEC], float (&acc)[VEC]) {
    if constexpr (DRES || sizeof(T) == 4) {
        // fp64 form: w*dy (exact in fp64), r*(wdy - x k) [+ dres] with one
        // final rounding.  Used when dx can cancel against dres, and for fp32
        // inputs, whose w*dy is not exact in fp32.
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const double wdy = (double)wc[k] * (double)dyv[k];
            const double t = __builtin_fma(-(double)xv[k], q.kk, wdy);
            if constexpr (DRES) o[k] = (float)__builtin_fma(q.r, t, (double)drv[k]);
            else o[k] = (float)(q.r * t);
            acc[k] += (dyv[k] * xv[k]) * q.rf;
        }
    } else {
        // bf16 inputs: w*dy is exact in fp32, and two fused multiply-adds
        // with k = k_hi + k_lo form wdy - x k to fp32 accuracy even where the
        // two terms nearly cancel.
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float wdy = wc[k] * dyv[k];
            float t = __builtin_fmaf(-xv[k], q.k_hi, wdy);
            t = __builtin_fmaf(-xv[k], q.k_lo, t);
            o[k] = q.rf * t;
            acc[k] += (dyv[k] * xv[k]) * q.rf;
        }
    }
}

}  // namespace rms
