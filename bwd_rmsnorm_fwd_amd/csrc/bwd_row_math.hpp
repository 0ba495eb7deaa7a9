// Per-row backward arithmetic shared by the backward row kernels (the
// register-tile, LDS-staged and streaming forms), and their cache hints.
//
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）":
//   §5.3 wdy = w*dy, c = (1/H) sum_j wdy_j x_j, dx = r (wdy - x r^2 c),
//   dw_j = sum over rows of dy_j x_j r.
#pragma once

#include <type_traits>

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

// Calls go(dres, rstd) with the two compile-time flags of a wide-row
// backward launch: a residual-stream gradient is added, and the saved rstd is
// read (else r is recomputed from x).  Fixing the second at compile time
// matters there: decided at run time, the recompute path's fp64 sums stay
// live beside the saved-rstd path's registers (the 512-lane streaming build
// at 65536 spilled 55 VGPRs, none now: bf16 1024 x 65536 row pass 131.4 ->
// 111.9 us).  The register tiles keep the run-time choice, which measured
// faster there (bf16 262144 x 128 row pass 34.9 vs 36.9 us).
template <typename Args, typename F>
__host__ inline void bwd_variant(const Args& a, F&& go) {
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (a.dres) {
        if (a.rstd) go(T_{}, T_{});
        else go(T_{}, F_{});
    } else {
        if (a.rstd) go(F_{}, T_{});
        else go(F_{}, F_{});
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int wait_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Sum over a team of TEAM lanes for kernels with direct-to-LDS loads in
// flight.  A fence before the barrier (even one restricted to LDS) would
// wait for those loads, so the slot write is waited for explicitly and the
// barrier stands alone, with compiler barriers keeping the LDS accesses on
// their side.  Slots as in team_sum_alt (callers alternate two sets).
template <int TEAM, typename V>
__device__ __forceinline__ V team_sum_nofence(V v, V* lds) {
    if constexpr (TEAM <= 64) {
        return team_sum_wave<TEAM>(v);
    } else {
        constexpr int NW = TEAM / kWave;
        v = team_sum_wave<64>(v);
        const int lt = threadIdx.x % TEAM;
        V* slot = lds + (threadIdx.x / TEAM) * NW;
        if ((lt & (kWave - 1)) == 0) slot[lt / kWave] = v;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's slot write is done
        asm volatile("" ::: "memory");           // no LDS access moves across
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        V s = slot[0];
#pragma unroll
        for (int k = 1; k < NW; ++k) s += slot[k];
        return s;
    }
}

// The workgroup's dw partial row from the column sums of its R = WG / TEAM
// teams (lane lt of a team holds columns (c * TEAM + lt) * VEC + k).  The
// teams are combined in team order through comb: side by side (summed per
// column) when that fits in 32 KiB, else one after another into a single
// row.  With VEC >= 4 the side-by-side layout is [team][chunk][group of four
// columns][lane] float4, so the lanes of a 128-bit LDS access are 16 bytes
// apart (no bank conflicts; the lane-major [team][column] layout put them 32
// bytes apart).  With VEC > 1, H is a multiple of VEC, so groups of four
// columns that start below H end below H; ldp is a multiple of 64.
template <int VEC, int TEAM, int NCH, int WG>
struct PartialComb {
    static constexpr int R = WG / TEAM;
    static constexpr int HT = TEAM * NCH * VEC;  // columns covered by one team
    static constexpr bool kWide = R > 1 && R * HT <= 8192;
    static constexpr int kFloats = R == 1 ? 1 : (kWide ? R * HT : HT);  // comb size
};

template <int VEC, int TEAM, int NCH, int WG>
__device__ __forceinline__ void write_partial(const float (&acc)[NCH][VEC], float* comb,
                                              float* prow, int H) {
    using PC = PartialComb<VEC, TEAM, NCH, WG>;
    constexpr int R = PC::R, HT = PC::HT;
    const int tid = threadIdx.x;
    const int team = tid / TEAM;
    const int lt = tid % TEAM;
    auto store4 = [&](int col, float a, float b, float c, float d) {
        u32x4 v;
        v.x = __float_as_uint(a); v.y = __float_as_uint(b);
        v.z = __float_as_uint(c); v.w = __float_as_uint(d);
        st128<false>(prow + col, v);
    };
    if constexpr (R == 1) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int col = (c * TEAM + lt) * VEC;
            if (col < H) {
                if constexpr (VEC == 1) {
                    prow[col] = acc[c][0];
                } else {
#pragma unroll
                    for (int k = 0; k < VEC; k += 4)
                        store4(col + k, acc[c][k], acc[c][k + 1], acc[c][k + 2], acc[c][k + 3]);
                }
            }
        }
    } else if constexpr (PC::kWide && VEC >= 4) {
        constexpr int NQ = VEC / 4;
        float4* c4 = reinterpret_cast<float4*>(comb);  // [R][NCH][NQ][TEAM]
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                c4[((team * NCH + c) * NQ + q) * TEAM + lt] =
                    make_float4(acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]);
        }
        __syncthreads();
        constexpr int NG = NCH * NQ * TEAM;  // float4 groups per team
        for (int i = tid; i < NG; i += WG) {
            const int c = i / (NQ * TEAM), q = (i / TEAM) % NQ, l = i % TEAM;
            const int col = (c * TEAM + l) * VEC + 4 * q;
            if (col < H) {
                float4 sum = c4[i];
                for (int t = 1; t < R; ++t) {
                    const float4 v = c4[t * NG + i];
                    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
                }
                store4(col, sum.x, sum.y, sum.z, sum.w);
            }
        }
    } else if constexpr (PC::kWide) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) comb[team * HT + (c * TEAM + lt) * VEC + k] = acc[c][k];
        }
        __syncthreads();
        for (int col = tid; col < H && col < HT; col += WG) {
            float sum = comb[col];
            for (int t = 1; t < R; ++t) sum += comb[t * HT + col];
            prow[col] = sum;
        }
    } else {
        for (int t = 0; t < R; ++t) {
            if (team == t) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const int col = (c * TEAM + lt) * VEC + k;
                        comb[col] = (t == 0) ? acc[c][k] : comb[col] + acc[c][k];
                    }
                }
            }
            __syncthreads();
        }
        if constexpr (VEC >= 4) {
            for (int col = tid * 4; col < H; col += WG * 4) {
                const float4 v = *reinterpret_cast<const float4*>(comb + col);
                store4(col, v.x, v.y, v.z, v.w);
            }
        } else {
            for (int col = tid; col < H && col < HT; col += WG) prow[col] = comb[col];
        }
    }
}

}  // namespace rms
