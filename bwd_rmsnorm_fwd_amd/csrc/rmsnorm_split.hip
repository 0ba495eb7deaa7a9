// Split-row forward for decode-sized batches (one or a few rows).
//
// P2 = trdm.cn/news/483216 (hand-written Triton decode kernels):
//   §3.2 split-K RMSNorm: several programs each sum the squares of one
//   segment of the row into a small partial array, then a merge step adds
//   the partials and a scale step applies r and the weight (fused here into
//   the merge, as P2 notes optimised versions do); §3.3 partials in fp32 and
//   a fixed-order merge rather than atomics; §5.1 the merge must not read
//   entries beyond the split count.
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）" §4.1
//   for the forward definition.
//
// Pass 1 (grid rows x splits, one wavefront each): chunk s of row i is
// columns [s*L, min((s+1)*L, H)) with L = ceil(H/splits) rounded up to the
// vector width; its sum of squares (exact fp32 squares of bf16 inputs,
// accumulated in fp64) is stored as one fp32 partial.
// Pass 2 (grid rows): adds the row's partials s = 0..splits-1 in order in
// fp64, forms r, writes rstd and y = (x * r) * w over the whole row.
#include "common.hpp"
#include "launch.hpp"

namespace rms {

template <typename T, int VEC>
__global__ __launch_bounds__(64) void split_sumsq_kernel(const T* __restrict__ x,
                                                         float* __restrict__ partials, int H,
                                                         int chunk, int splits) {
    const int64_t row = blockIdx.x;
    const int s = blockIdx.y;
    const T* xr = x + row * (int64_t)H;
    const int c0 = s * chunk;
    const int c1 = c0 + chunk < H ? c0 + chunk : H;
    double ss = 0.0;
    for (int col = c0 + (int)threadIdx.x * VEC; col < c1; col += 64 * VEC) {
        float v[VEC];
        unpack(load_pack<T, VEC>(xr + col), v);
#pragma unroll
        for (int k = 0; k < VEC; ++k) ss += sq64(v[k], (T*)nullptr);
    }
    ss = team_sum_wave<64>(ss);
    if (threadIdx.x == 0) partials[row * splits + s] = (float)ss;
}

template <typename T, int VEC, int WG>
__global__ __launch_bounds__(WG) void split_finalize_kernel(const T* __restrict__ x,
                                                            const T* __restrict__ w,
                                                            const float* __restrict__ partials,
                                                            T* __restrict__ y,
                                                            float* __restrict__ rstd, int H,
                                                            int splits, float eps) {
    const int64_t row = blockIdx.x;
    const float* pr = partials + row * splits;
    double ss = 0.0;
    for (int s = 0; s < splits; ++s) ss += (double)pr[s];  // index order, never past `splits`
    const double r = rsqrt_f64(ss * (1.0 / (double)H) + (double)eps);
    const float rf = (float)r;
    if (threadIdx.x == 0 && rstd) rstd[row] = rf;
    const T* xr = x + row * (int64_t)H;
    T* yr = y + row * (int64_t)H;
    for (int col = (int)threadIdx.x * VEC; col < H; col += WG * VEC) {
        float v[VEC], wv[VEC], o[VEC];
        unpack(load_pack<T, VEC>(xr + col), v);
        unpack(load_pack<T, VEC>(w + col), wv);
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = (v[k] * rf) * wv[k];
        store_vec<T, VEC>(yr + col, o);
    }
}

template <typename T, int VEC>
static hipError_t launch_split(const FwdArgs& a, float* partials, int splits, hipStream_t s) {
    const int n = (a.H + VEC - 1) / VEC;
    const int chunk = ((n + splits - 1) / splits) * VEC;
    RMS_LAUNCH((split_sumsq_kernel<T, VEC>), dim3((unsigned)a.rows, splits), dim3(64), 0, s,
                       (const T*)a.x, partials, a.H, chunk, splits);
    hipError_t e = launch_error();
    if (e != hipSuccess) return e;
    RMS_LAUNCH((split_finalize_kernel<T, VEC, 128>), dim3((unsigned)a.rows), dim3(128), 0, s,
                       (const T*)a.x, (const T*)a.w, (const float*)partials, (T*)a.y, a.rstd, a.H,
                       splits, a.eps);
    return launch_error();
}

hipError_t launch_splitrow(DType dt, int vec, const FwdArgs& a, float* partials, int splits,
                           hipStream_t s) {
    if (dt == DType::F32) {
        return vec == 4 ? launch_split<float, 4>(a, partials, splits, s)
                        : launch_split<float, 1>(a, partials, splits, s);
    }
    return vec == 8 ? launch_split<bf16_t, 8>(a, partials, splits, s)
                    : launch_split<bf16_t, 1>(a, partials, splits, s);
}

}  // namespace rms
