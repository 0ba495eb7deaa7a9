// Backward RMSNorm for gfx950: a row pass (dx and per-workgroup dw partial
// column sums) and a dw reduce pass.
//
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）":
//   §5.3 wdy = w*dy, c = (1/H) sum_j wdy_j x_j, dx = r (wdy - x r^2 c),
//   dw_j = sum over rows of dy_j x_j r; §5.4 dw in two passes (per-program
//   partials, then a cross-row sum) rather than atomics, whose ordering makes
//   results jitter; §5.6 reductions in fp32, not bf16.
// P2 = trdm.cn/news/483216: §3.3 fixed-order merge of fp32 partials for
//   run-to-run reproducibility.
//
// Design (MI355X):
//   * Row pass: G persistent workgroups; rows go in blocks of R (one team
//     per row, as in the forward) dealt round-robin to the workgroups, each
//     prefetching its next block while finishing the current one.
//     dy, x (and dres) are read once, through buffer resources sized to the
//     block's rows; rstd is the forward's saved statistic (or is recomputed
//     from x when none is given).  Rows of 1024-lane teams with two chunks
//     per lane stage the next row in LDS instead of registers
//     (bwd_rows_staged_kernel); wider rows are held in LDS one at a time
//     where x and dy fit (bwd_rows_ldsrow_kernel), else streamed twice, one
//     row per workgroup (bwd_rows_wide_kernel).
//   * The row sums c (and sum x^2 when recomputing) are exact fp32 products
//     (for bf16 inputs) accumulated in fp64, so c and r carry no cancellation
//     error.  dx uses k = r^2 c split into two floats, k_hi + k_lo, applied
//     with two fused multiply-adds: wdy - x k is formed with one rounding,
//     which keeps dx accurate where its two terms nearly cancel.
//   * dw: each lane keeps fp32 column sums for its columns over the
//     workgroup's rows; the R teams are combined through LDS in team order,
//     and the workgroup writes one partial row.  The reduce pass adds the G
//     partial rows per column in a fixed order.  No atomics anywhere.
#include "bwd_row_math.hpp"
#include "launch.hpp"

// 1: the next row block loads while the current one is finished (two
// register sets in turn); 0: one block at a time.
#ifndef RMS_BWD_PREFETCH
#define RMS_BWD_PREFETCH 1
#endif

namespace rms {

template <typename T, int VEC, int TEAM, int NCH, int WG, bool DRES>
__global__ __launch_bounds__(WG) void bwd_rows_kernel(const T* dy, const T* __restrict__ x,
                                                      const T* __restrict__ w,
                                                      const float* __restrict__ rstd,
                                                      const T* dres, T* dx,
                                                      float* __restrict__ partial, int64_t rows,
                                                      int H, int ldp, float eps) {
    constexpr int R = WG / TEAM;
    constexpr int NWT = TEAM > kWave ? TEAM / kWave : 1;
    constexpr int EB = NCH * VEC * (int)sizeof(T);  // bytes per lane per row tensor
    // Register budget: w cached and the next rows prefetched unless the
    // per-lane tile is large for this workgroup size.
    constexpr bool kCacheW = EB * WG <= 16384;
    constexpr bool kPrefetch = RMS_BWD_PREFETCH != 0 && EB * WG <= 16384;
    constexpr bool kNtLoad = DRES ? RMS_DRES_NT_LOAD != 0 : RMS_BWD_NT_LOAD != 0;
    constexpr bool kNtStore = DRES ? RMS_DRES_NT_STORE != 0 : RMS_BWD_NT_STORE != 0;
    // Row-sum slots: two sets used in turn (one barrier per sum), each
    // with room for c and, when recomputing r, sum x^2.
    constexpr int kRedSet = 2 * R * NWT;
    __shared__ double red[TEAM > kWave ? 2 * kRedSet : 1];
    __shared__ __align__(16) float comb[PartialComb<VEC, TEAM, NCH, WG>::kFloats];

    const int tid = threadIdx.x;
    const int team = tid / TEAM;
    const int lt = tid % TEAM;
    const bool has_rstd = rstd != nullptr;
    const double inv_h = 1.0 / (double)H;  // exact for power-of-two H
    // Row blocks of R rows are dealt round-robin: workgroup g takes blocks
    // g, g + G, g + 2G, ..., so at any moment the workgroups stream
    // neighbouring rows (measured 5-9% faster than contiguous row ranges per
    // workgroup, which scatter the concurrent streams across memory).
    const int64_t begin = (int64_t)blockIdx.x * R;
    const int64_t stride = (int64_t)gridDim.x * R;
    const int64_t end = rows;

    float wv[kCacheW ? NCH : 1][VEC];
    float acc[NCH][VEC];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if constexpr (kCacheW) {
            const int col = (c * TEAM + lt) * VEC;
            Pack<T, VEC> p = col < H ? load_pack<T, VEC>(w + col) : zero_pack<T, VEC>();
            unpack(p, wv[c]);
        }
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
    }
    auto weights = [&](int c, float (&wc)[VEC]) {
        if constexpr (kCacheW) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) wc[k] = wv[c][k];
        } else {
            const int col = (c * TEAM + lt) * VEC;
            unpack(col < H ? load_pack<T, VEC>(w + col) : zero_pack<T, VEC>(), wc);
        }
    };

    // One row block's operands, read through buffer resources sized to the
    // rows of the block that exist: lanes of rows past the end, and lanes of
    // columns past H (offset kBufOutside), load zeros and their stores are
    // dropped.  Every lane issues the same loads on every path, so the
    // compiler waits for exactly the block it is about to use while the
    // next block's loads stay in flight.
    struct Blk {
        Pack<T, VEC> x[NCH], dy[NCH], dr[DRES ? NCH : 1];
        float rs;
    };
    uint32_t voff[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * TEAM + lt) * VEC;
        voff[c] = col < H ? (uint32_t)(team * H + col) * (uint32_t)sizeof(T) : kBufOutside;
    }
    auto block_rows = [&](int64_t b) -> uint32_t {  // rows of block b that exist (b < end)
        return (uint32_t)(end - b < R ? end - b : R);
    };
    auto issue = [&](int64_t b, Blk& q) {
        const int64_t off = b * (int64_t)H;
        const uint32_t nr = block_rows(b);
        const uint32_t bytes = nr * (uint32_t)H * (uint32_t)sizeof(T);
        const BufRes rx = buf_rsrc(x + off, bytes);
        const BufRes rdy = buf_rsrc(dy + off, bytes);
        const BufRes rdr = buf_rsrc(DRES ? dres + off : x, DRES ? bytes : 0u);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            q.x[c] = buf_load_pack<T, VEC, kNtLoad>(rx, voff[c]);
            q.dy[c] = buf_load_pack<T, VEC, kNtLoad>(rdy, voff[c]);
            if constexpr (DRES) q.dr[c] = buf_load_pack<T, VEC, kNtLoad>(rdr, voff[c]);
        }
        // Without a saved statistic the resource is empty (size 0), so the
        // load returns zero and reads nothing.
        const BufRes rr = has_rstd ? buf_rsrc(rstd + b, nr * 4u) : buf_rsrc(x, 0u);
        q.rs = buf_load_f32(rr, (uint32_t)team * 4u);
    };

    auto process = [&](int64_t b, Blk& q, int set) {
        const int64_t row = b + team;
        const bool active = row < end;
        // Pass A: row sums.  Values are unpacked again in pass B rather than
        // kept live across the reduction (unpacking is a shift or a mask).
        double cs = 0.0, ss = 0.0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float xv[VEC], dyv[VEC], wc[VEC];
            unpack(q.x[c], xv);
            unpack(q.dy[c], dyv);
            weights(c, wc);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                cs += prod3_64(wc[k], dyv[k], xv[k], (T*)nullptr);
                if (!has_rstd) ss += sq64(xv[k], (T*)nullptr);
            }
        }
        double* rs_slots = red + (TEAM > kWave ? set * kRedSet : 0);
        cs = team_sum_alt<TEAM>(cs, rs_slots);
        double r;
        if (has_rstd) {
            r = (double)q.rs;
        } else {
            ss = team_sum_alt<TEAM>(ss, rs_slots + R * NWT);
            r = rsqrt_f64(ss * inv_h + (double)eps);
        }
        const RowK kq = row_k(r, cs, inv_h, active);
        // Pass B: dx and the dw column sums.
        const BufRes rdx = buf_rsrc(dx + b * (int64_t)H,
                                    block_rows(b) * (uint32_t)H * (uint32_t)sizeof(T));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float xv[VEC], dyv[VEC], wc[VEC], drv[VEC], o[VEC];
            unpack(q.x[c], xv);
            unpack(q.dy[c], dyv);
            weights(c, wc);
            if constexpr (DRES) unpack(q.dr[c], drv);
            dx_chunk<T, VEC, DRES>(xv, dyv, wc, drv, kq, o, acc[c]);
            buf_store_vec<T, VEC, kNtStore, DRES>(rdx, voff[c], o);
        }
    };

    if constexpr (kPrefetch) {
        // Two register sets in turn: block b + stride loads while block b is
        // finished.  The last one or two blocks are peeled off the loop so
        // that nothing is loaded past the workgroup's last block.
        const int64_t nb = begin < end ? (end - begin + stride - 1) / stride : 0;
        Blk A, B;
        int64_t b = begin;
        if (nb > 0) {
            issue(b, A);
            int64_t left = nb;
            while (left > 2) {
                issue(b + stride, B);
                process(b, A, 0);
                b += stride;
                issue(b + stride, A);
                process(b, B, 1);
                b += stride;
                left -= 2;
            }
            if (left == 2) {
                issue(b + stride, B);
                process(b, A, 0);
                process(b + stride, B, 1);
            } else {
                process(b, A, 0);
            }
        }
    } else {
        Blk A;
        int set = 0;
        for (int64_t b = begin; b < end; b += stride) {
            issue(b, A);
            process(b, A, set);
            set ^= 1;
        }
    }
    // One partial row per workgroup: the R teams combined in team order.
    write_partial<VEC, TEAM, NCH, WG>(acc, comb, partial + (int64_t)blockIdx.x * ldp, H);
}

// dw[j] = sum_{g < G} partial[g][j] in a fixed order.  A workgroup of
// kRedWG lanes owns kRedCols = 32 columns: lane t takes the four columns
// 4 (t % 8) .. + 3 (one 128-bit load per partial row) and the partial rows
// g = gl, gl + 32, gl + 64, ... with gl = t / 8, adding them in increasing g
// with all of its loads in flight at once (rows past G load as zero, which
// leaves the sum unchanged).  The 32 gl sums of a column are then added as a
// tree: across the 8 gl of a wavefront by lane exchanges (xor 8, 16, 32:
// both partners form the same sum, a + b == b + a), then the 4 wavefronts'
// sums through LDS in wave order.  The order depends on G alone.
#ifndef RMS_RED_UNROLL
#define RMS_RED_UNROLL 8
#endif
constexpr int kRedWG = 256;
constexpr int kRedCL = 8;                  // column lanes (4 columns each)
constexpr int kRedGL = kRedWG / kRedCL;    // 32 partial-row lanes
constexpr int kRedCols = 4 * kRedCL;       // 32 columns per workgroup
constexpr int kRedU = RMS_RED_UNROLL;
static_assert(64 % kRedCols == 0, "reduce tile must divide ldp (multiple of 64)");

__device__ __forceinline__ float shfl_xor_f32(float v, int m) {
    const int src = (int)(threadIdx.x % kWave) ^ m;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

template <typename T>
__global__ __launch_bounds__(kRedWG) void dw_reduce_kernel(const float* __restrict__ partial, int G,
                                                           int ldp, int H, T* __restrict__ dw) {
    __shared__ float4 part[kRedWG / kWave][kRedCL];
    const int cl = threadIdx.x % kRedCL;
    const int gl = threadIdx.x / kRedCL;
    // ldp is a multiple of 64 and of kRedCols, so col0 + 3 < ldp for every workgroup.
    const int col0 = blockIdx.x * kRedCols + cl * 4;
    const float* base = partial + col0;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int g = gl; g < G; g += kRedU * kRedGL) {
        float4 p[kRedU];
#pragma unroll
        for (int u = 0; u < kRedU; ++u) {
            const int gu = g + u * kRedGL;
            p[u] = gu < G ? *reinterpret_cast<const float4*>(base + (int64_t)gu * ldp)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kRedU; ++u) { a.x += p[u].x; a.y += p[u].y; a.z += p[u].z; a.w += p[u].w; }
    }
    // Lanes cl + 8 j (j = 0..7) of a wavefront hold the same columns.
#pragma unroll
    for (int m = 8; m < kWave; m <<= 1) {
        a.x += shfl_xor_f32(a.x, m);
        a.y += shfl_xor_f32(a.y, m);
        a.z += shfl_xor_f32(a.z, m);
        a.w += shfl_xor_f32(a.w, m);
    }
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) < kRedCL) part[wave][cl] = a;
    __syncthreads();
    if (threadIdx.x < kRedCols) {
        const int c4 = threadIdx.x / 4, k = threadIdx.x % 4;
        const float* p0 = reinterpret_cast<const float*>(&part[0][c4]);
        float sum = p0[k];
#pragma unroll
        for (int v = 1; v < kRedWG / kWave; ++v) sum += reinterpret_cast<const float*>(&part[v][c4])[k];
        const int col = blockIdx.x * kRedCols + threadIdx.x;
        if (col < H) {
            float o[1] = {sum};
            store_vec<T, 1>(dw + col, o);
        }
    }
}

#ifndef RMS_BWD_MAX_GROUPS
#define RMS_BWD_MAX_GROUPS 256
#endif
#ifndef RMS_BWD_MIN_ROWS_PER_GROUP
#define RMS_BWD_MIN_ROWS_PER_GROUP 4
#endif

int bwd_groups(int64_t rows, int64_t H, DType) {
    // One workgroup per CU on every tile (a pure function of the shape, so
    // the reduction order and the bits of dw depend on nothing else).
    (void)H;
    if (rows <= 0) return 0;
    const int64_t n = (rows + RMS_BWD_MIN_ROWS_PER_GROUP - 1) / RMS_BWD_MIN_ROWS_PER_GROUP;
    return (int)(n < RMS_BWD_MAX_GROUPS ? n : RMS_BWD_MAX_GROUPS);
}

int partial_ld(int64_t H) { return (int)((H + 63) / 64 * 64); }

template <typename T, int VEC, int TEAM, int NCH>
static hipError_t launch_rows_cfg(const BwdArgs& a, hipStream_t s) {
    // Workgroup size by bytes per lane (EB): 512 lanes, shared among several
    // rows by narrow tiles, and 256 for tiles of more than 32 bytes per lane
    // so that the row, its prefetched successor, w and the dw sums stay in
    // registers.  Teams wider than that fill the workgroup alone, and a
    // one-chunk team of 512 lanes or more is a workgroup of its own.
    // 1024-lane groups for the narrow tiles measured slower (bf16 262144 x
    // 128 row pass 36.0 -> 34.5 us with 512 lanes; with a residual-stream
    // gradient, whose 1024-lane form spilled in the row loop, 51.2 -> 47.9).
    constexpr int EB = NCH * VEC * (int)sizeof(T);
    constexpr int WGD = (TEAM >= 512 && NCH == 1) ? TEAM : (EB <= 32 ? 512 : 256);
    constexpr int WG = TEAM > WGD ? TEAM : WGD;
    if (a.dres) {
        RMS_LAUNCH((bwd_rows_kernel<T, VEC, TEAM, NCH, WG, true>), dim3(a.G), dim3(WG), 0,
                           s, (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd,
                           (const T*)a.dres, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    } else {
        RMS_LAUNCH((bwd_rows_kernel<T, VEC, TEAM, NCH, WG, false>), dim3(a.G), dim3(WG), 0,
                           s, (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd,
                           (const T*)nullptr, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    }
    return launch_error();
}

template <typename T, int VEC>
static hipError_t dispatch_rows(const BwdArgs& a, hipStream_t s) {
    Geometry g;
    if (!choose_geometry(a.H, VEC, a.dres != nullptr, &g)) return hipErrorInvalidValue;
    const DType dt = sizeof(T) == 4 ? DType::F32 : DType::BF16;
    if (g.team == 1024 && g.nch >= 4) return launch_bwd_wide(dt, VEC, a, s);
    if (VEC > 1 && g.team == 1024 && g.nch == 2) return launch_bwd_staged(dt, VEC, a, s);
#define RMS_CASE(TM, NC) \
    if (g.team == TM && g.nch == NC) return launch_rows_cfg<T, VEC, TM, NC>(a, s);
    RMS_CASE(1, 1) RMS_CASE(2, 1) RMS_CASE(4, 1) RMS_CASE(8, 1) RMS_CASE(16, 1) RMS_CASE(32, 1)
    RMS_CASE(64, 1) RMS_CASE(64, 2) RMS_CASE(128, 2) RMS_CASE(256, 2) RMS_CASE(512, 1)
    RMS_CASE(512, 2)
    // With 128-bit access the 1024 x 2 tile goes to the LDS-staged kernel
    // above, so the register tile is built for the scalar path only.
    if constexpr (VEC == 1) { RMS_CASE(1024, 2) }
#undef RMS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_rows(DType dt, int vec, const BwdArgs& a, hipStream_t s) {
    if (dt == DType::F32) {
        return vec == 4 ? dispatch_rows<float, 4>(a, s) : dispatch_rows<float, 1>(a, s);
    }
    return vec == 8 ? dispatch_rows<bf16_t, 8>(a, s) : dispatch_rows<bf16_t, 1>(a, s);
}

hipError_t launch_dw_reduce(DType dt, const float* partial, int G, int ldp, int H, void* dw,
                            hipStream_t s) {
    const int grid = ldp / kRedCols;
    if (dt == DType::F32) {
        RMS_LAUNCH((dw_reduce_kernel<float>), dim3(grid), dim3(kRedWG), 0, s, partial, G, ldp,
                           H, (float*)dw);
    } else {
        RMS_LAUNCH((dw_reduce_kernel<bf16_t>), dim3(grid), dim3(kRedWG), 0, s, partial, G, ldp,
                           H, (bf16_t*)dw);
    }
    return launch_error();
}

}  // namespace rms
