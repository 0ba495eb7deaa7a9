// Split-K matrix-vector product for decode (one input row), gfx950.
//
// P2 = trdm.cn/news/483216 (hand-written Triton decode kernels): §3.1 at
//   batch 1 every projection is a matrix-vector product; a program per output
//   block loops serially over the whole reduction dimension K and leaves the
//   GPU idle, so K is cut into SPLIT_K segments reduced in parallel into an
//   fp32 partial buffer and merged by a separate reduce kernel
//   (splitk_reduce); §3.3 partials stay fp32 and the merge runs in a fixed
//   order, not with atomics; §5.1 the merge must not read past the split count.
//
// y[n] = sum_k A[n][k] x[k], A row-major [N][K].
// Pass 1 (grid ceil(N / RPW) x S, 256 lanes): a team of TEAM lanes owns row n
//   within segment s = [s*L, min((s+1)*L, K)), L = ceil(K/S) rounded up to the
//   vector width; lanes stride the segment with 128-bit loads (A streamed with
//   nontemporal loads, x through the caches), products accumulate in fp64
//   (exact fp32 products for bf16 inputs), the team reduces with DPP.  With
//   S == 1 the team writes y[n] directly; otherwise partials[s*N + n] (fp32).
// Pass 2 (splitk_reduce, one lane per n): adds partials s = 0..S-1 in index
//   order in fp64 and rounds once to the output dtype.
#include "common.hpp"
#include "launch.hpp"

namespace rms {

template <typename T, int VEC, int TEAM>
__global__ __launch_bounds__(256) void gemv_splitk_kernel(const T* __restrict__ A,
                                                          const T* __restrict__ x,
                                                          T* __restrict__ y,
                                                          float* __restrict__ partials, int N,
                                                          int K, int seg, int splits) {
    constexpr int RPW = 256 / TEAM;
    const int team = threadIdx.x / TEAM;
    const int lt = threadIdx.x % TEAM;
    const int n = blockIdx.x * RPW + team;
    const int s = blockIdx.y;
    const int k0 = s * seg;
    const int k1 = k0 + seg < K ? k0 + seg : K;
    double acc = 0.0;
    if (n < N) {
        const T* a = A + (int64_t)n * K;
        int k = k0 + lt * VEC;
        // Four independent 128-bit loads in flight per lane, then the rest.
        for (; k + 3 * TEAM * VEC < k1; k += 4 * TEAM * VEC) {
            Pack<T, VEC> pa[4], px[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pa[u] = load_pack<T, VEC, true>(a + k + u * TEAM * VEC);
                px[u] = load_pack<T, VEC>(x + k + u * TEAM * VEC);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float av[VEC], xv[VEC];
                unpack(pa[u], av);
                unpack(px[u], xv);
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc += prod2_64(av[v], xv[v], (T*)nullptr);
            }
        }
        for (; k < k1; k += TEAM * VEC) {
            float av[VEC], xv[VEC];
            unpack(load_pack<T, VEC, true>(a + k), av);
            unpack(load_pack<T, VEC>(x + k), xv);
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc += prod2_64(av[v], xv[v], (T*)nullptr);
        }
    }
    acc = team_sum_wave<TEAM>(acc);
    if (n < N && lt == 0) {
        if (splits == 1) {
            float o[1] = {(float)acc};
            store_vec<T, 1>(y + n, o);
        } else {
            partials[(int64_t)s * N + n] = (float)acc;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials,
                                                            T* __restrict__ y, int N, int splits) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    double acc = 0.0;
    for (int s = 0; s < splits; ++s) acc += (double)partials[(int64_t)s * N + n];
    float o[1] = {(float)acc};
    store_vec<T, 1>(y + n, o);
}

template <typename T, int VEC, int TEAM>
static hipError_t launch_team(const GemvArgs& a, hipStream_t st) {
    constexpr int RPW = 256 / TEAM;
    const dim3 grid((unsigned)((a.N + RPW - 1) / RPW), (unsigned)a.splits);
    RMS_LAUNCH((gemv_splitk_kernel<T, VEC, TEAM>), grid, dim3(256), 0, st, (const T*)a.A,
                       (const T*)a.x, (T*)a.y, a.partials, a.N, a.K, a.seg, a.splits);
    hipError_t e = launch_error();
    if (e != hipSuccess || a.splits == 1) return e;
    RMS_LAUNCH((splitk_reduce_kernel<T>), dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0,
                       st, (const float*)a.partials, (T*)a.y, a.N, a.splits);
    return launch_error();
}

template <typename T, int VEC>
static hipError_t dispatch_gemv(const GemvArgs& a, hipStream_t st) {
    switch (a.team) {
        case 1: return launch_team<T, VEC, 1>(a, st);
        case 2: return launch_team<T, VEC, 2>(a, st);
        case 4: return launch_team<T, VEC, 4>(a, st);
        case 8: return launch_team<T, VEC, 8>(a, st);
        case 16: return launch_team<T, VEC, 16>(a, st);
        case 32: return launch_team<T, VEC, 32>(a, st);
        case 64: return launch_team<T, VEC, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(DType dt, int vec, const GemvArgs& a, hipStream_t st) {
    if (dt == DType::F32) {
        return vec == 4 ? dispatch_gemv<float, 4>(a, st) : dispatch_gemv<float, 1>(a, st);
    }
    return vec == 8 ? dispatch_gemv<bf16_t, 8>(a, st) : dispatch_gemv<bf16_t, 1>(a, st);
}

}  // namespace rms
