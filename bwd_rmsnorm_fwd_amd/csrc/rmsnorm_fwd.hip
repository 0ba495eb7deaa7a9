// Forward RMSNorm and residual-add + RMSNorm row kernels for gfx950.
//
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）":
//   §4.1 y = w * x / sqrt(mean(x^2) + eps) per row; §4.2 one program per row,
//   fp32 upcast, masked tail contributing zero, mean over the true width.
// P2 = trdm.cn/news/483216 (hand-written Triton decode kernels): §2.1 the
//   residual_add -> rms_norm pair and the fused kernel planned there.
//
// Design (MI355X): a team of TEAM lanes owns a row (several rows per
// wavefront for narrow H, a whole workgroup for wide H); the row stays in
// registers between the sum of squares and the scaled store, so x is read
// from HBM exactly once.  Loads/stores are 128-bit per lane and contiguous
// across the team.  The sum of squares is exact-product fp32 accumulated in
// fp64 per lane, reduced with DPP inside 16-lane rows and lane reads across
// rows (LDS across wavefronts).  The grid has one workgroup per row block up
// to RMS_FWD_MAX_GRID workgroups; beyond that a workgroup takes several
// blocks and prefetches the next while finishing the current one.
#include "common.hpp"
#include "launch.hpp"

// Grid size: ceil(bytes of x / RMS_FWD_WG_BYTES), at least RMS_FWD_MIN_GRID
// and at most one workgroup per row block.  Measured: one block per
// workgroup is best at every width (bf16 residual 16384 x 4096: 87 vs 92 us
// against a fixed 4096-workgroup grid; bf16 262144 x 128, 4 KB blocks: 23.2
// -> 23.0 us for one block per workgroup instead of two).
#ifndef RMS_FWD_WG_BYTES
#define RMS_FWD_WG_BYTES 4096
#endif
#ifndef RMS_FWD_MIN_GRID
#define RMS_FWD_MIN_GRID 2048
#endif
#ifndef RMS_FWD_MAX_GRID
#define RMS_FWD_MAX_GRID (1 << 20)
#endif
// Streaming (nontemporal) access to the row tensors: x/res loads, y/h
// stores.  Measured best with inputs that are not in the Infinity Cache:
// loads and stores (cached loads: bf16 4096 x 4096 12.4 -> 13.5 us, 262144
// x 128 23.3 -> 24.2, 8192 x 8192 44.0 -> 45.2; the residual forward at
// 16384 x 4096 84.1 -> 88.1).
#ifndef RMS_FWD_NT_LOAD
#define RMS_FWD_NT_LOAD 1
#endif
#ifndef RMS_FWD_NT_STORE
#define RMS_FWD_NT_STORE 1
#endif
#ifndef RMS_RESFWD_NT_LOAD
#define RMS_RESFWD_NT_LOAD 1
#endif
#ifndef RMS_RESFWD_NT_STORE
#define RMS_RESFWD_NT_STORE 1
#endif
// Row blocks in flight per workgroup beyond the one being finished (1 or 2).
#ifndef RMS_FWD_PREFETCH
#define RMS_FWD_PREFETCH 1
#endif

namespace rms {

template <typename T, int VEC, int TEAM, int NCH, int WG, bool RES>
__global__ __launch_bounds__(WG) void fwd_kernel(const T* x, const T* res, const T* __restrict__ w,
                                                 T* h, T* __restrict__ y,
                                                 float* __restrict__ rstd, int64_t rows, int H,
                                                 float eps) {
    constexpr int R = WG / TEAM;  // rows per workgroup iteration
    constexpr int NWT = TEAM > kWave ? TEAM / kWave : 1;
    // Register budget: keep w and a prefetched row in registers unless the
    // per-lane tile is large for this workgroup size.
    constexpr int E = NCH * VEC;
    constexpr bool kCacheW = E * WG <= 32768;
    constexpr bool kPrefetch = E * WG <= 32768;
    constexpr bool kNtLoad = RES ? RMS_RESFWD_NT_LOAD != 0 : RMS_FWD_NT_LOAD != 0;
    constexpr bool kNtStore = RES ? RMS_RESFWD_NT_STORE != 0 : RMS_FWD_NT_STORE != 0;
    constexpr int kDepth = kPrefetch ? RMS_FWD_PREFETCH : 0;
    // Row-sum slots: two sets used by alternate row blocks (one barrier per
    // sum; a set is rewritten only after the barrier of the block between).
    __shared__ double red[TEAM > kWave ? 2 * R * NWT : 1];

    const int tid = threadIdx.x;
    const int team = tid / TEAM;
    const int lt = tid % TEAM;
    const int64_t nrb = (rows + R - 1) / R;
    const double inv_h = 1.0 / (double)H;  // exact for power-of-two H

    float wv[kCacheW ? NCH : 1][VEC];
    if constexpr (kCacheW) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int col = (c * TEAM + lt) * VEC;
            Pack<T, VEC> p = col < H ? load_pack<T, VEC>(w + col) : zero_pack<T, VEC>();
            unpack(p, wv[c]);
        }
    }

    // Row blocks are read and written through buffer resources sized to the
    // block's rows that exist; lanes of rows past the end, and of columns
    // past H (offset kBufOutside), load zeros and their stores are dropped.
    struct RowRegs {
        Pack<T, VEC> x[NCH], r[RES ? NCH : 1];
    };
    uint32_t voff[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * TEAM + lt) * VEC;
        voff[c] = col < H ? (uint32_t)(team * H + col) * (uint32_t)sizeof(T) : kBufOutside;
    }
    auto block_bytes = [&](int64_t rb) -> uint32_t {  // bytes of block rb's rows (rb < nrb)
        const int64_t left = rows - rb * R;
        return (uint32_t)(left < R ? left : R) * (uint32_t)H * (uint32_t)sizeof(T);
    };
    auto load_row = [&](int64_t rb, RowRegs& q) {
        const int64_t off = rb * R * (int64_t)H;
        const uint32_t bytes = block_bytes(rb);
        const BufRes rx = buf_rsrc(x + off, bytes);
        const BufRes rr = buf_rsrc(RES ? res + off : x, RES ? bytes : 0u);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            q.x[c] = buf_load_pack<T, VEC, kNtLoad>(rx, voff[c]);
            if constexpr (RES) q.r[c] = buf_load_pack<T, VEC, kNtLoad>(rr, voff[c]);
        }
    };

    // Ring of row blocks in flight: cur is being finished, ahead[d] is block
    // rb + (d + 1) * gridDim.x (loads issued kDepth blocks ahead).
    RowRegs cur;
    RowRegs ahead[kDepth > 0 ? kDepth : 1];
    int64_t rb = blockIdx.x;
    if constexpr (kDepth > 0) {
        if (rb < nrb) load_row(rb, cur);
#pragma unroll
        for (int d = 0; d + 1 < kDepth; ++d) {
            const int64_t b = rb + (d + 1) * (int64_t)gridDim.x;
            if (b < nrb) load_row(b, ahead[d]);
        }
    }
    int set = 0;  // row-sum slot set of this block
    while (rb < nrb) {
        const int64_t nb = rb + gridDim.x;
        if constexpr (kDepth > 0) {
            const int64_t fb = rb + kDepth * (int64_t)gridDim.x;
            if (fb < nrb) load_row(fb, ahead[kDepth - 1]);
        } else {
            load_row(rb, cur);
        }

        const int64_t row = rb * R + team;
        const bool active = row < rows;
        const int64_t boff = rb * R * (int64_t)H;
        const uint32_t bbytes = block_bytes(rb);
        const BufRes ry = buf_rsrc(y + boff, bbytes);
        const BufRes rh = buf_rsrc(RES ? h + boff : y, RES ? bbytes : 0u);
        float v[NCH][VEC];
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            unpack(cur.x[c], v[c]);
            if constexpr (RES) {
                float rv[VEC];
                unpack(cur.r[c], rv);
#pragma unroll
                for (int k = 0; k < VEC; ++k) v[c][k] = round_to(v[c][k] + rv[k], (T*)nullptr);
                buf_store_vec<T, VEC, kNtStore>(rh, voff[c], v[c]);
            }
#pragma unroll
            for (int k = 0; k < VEC; ++k) ss += sq64(v[c][k], (T*)nullptr);
        }
        ss = team_sum_alt<TEAM>(ss, red + (TEAM > kWave ? set * R * NWT : 0));
        const double r = rsqrt_f64(ss * inv_h + (double)eps);
        const float rf = (float)r;
        if (active && lt == 0 && rstd) rstd[row] = rf;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int col = (c * TEAM + lt) * VEC;
            float wc[VEC], o[VEC];
            if constexpr (kCacheW) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) wc[k] = wv[c][k];
            } else {
                unpack(col < H ? load_pack<T, VEC>(w + col) : zero_pack<T, VEC>(), wc);
            }
#pragma unroll
            for (int k = 0; k < VEC; ++k) o[k] = (v[c][k] * rf) * wc[k];
            buf_store_vec<T, VEC, kNtStore>(ry, voff[c], o);
        }

        if constexpr (kDepth > 0) {
            cur = ahead[0];
#pragma unroll
            for (int d = 0; d + 1 < kDepth; ++d) ahead[d] = ahead[d + 1];
        }
        rb = nb;
        set ^= 1;
    }
}

template <typename T, int VEC, int TEAM, int NCH>
static hipError_t launch_cfg(const FwdArgs& a, bool residual, hipStream_t s) {
    // 256 lanes, or the team if wider; one-chunk teams of up to 64 lanes
    // (rows of 1 KB or less) take 512 so that a row block is 8 KB (measured
    // on bf16 262144 x 128: forward 22.5 -> 21.9 us; 1024 lanes 21.9 but
    // slower inside the fwd + bwd step).
    constexpr int WG = TEAM > 256 ? TEAM : ((TEAM <= 64 && NCH == 1) ? 512 : 256);
    constexpr int R = WG / TEAM;
    const int64_t nrb = (a.rows + R - 1) / R;
    const int64_t xbytes = a.rows * (int64_t)a.H * (int64_t)sizeof(T);
    int64_t want = (xbytes + RMS_FWD_WG_BYTES - 1) / RMS_FWD_WG_BYTES;
    if (want < RMS_FWD_MIN_GRID) want = RMS_FWD_MIN_GRID;
    if (want > RMS_FWD_MAX_GRID) want = RMS_FWD_MAX_GRID;
    const int grid = (int)(nrb < want ? nrb : want);
    if (residual) {
        RMS_LAUNCH((fwd_kernel<T, VEC, TEAM, NCH, WG, true>), dim3(grid), dim3(WG), 0, s,
                           (const T*)a.x, (const T*)a.res, (const T*)a.w, (T*)a.h, (T*)a.y, a.rstd,
                           a.rows, a.H, a.eps);
    } else {
        RMS_LAUNCH((fwd_kernel<T, VEC, TEAM, NCH, WG, false>), dim3(grid), dim3(WG), 0, s,
                           (const T*)a.x, (const T*)nullptr, (const T*)a.w, (T*)nullptr, (T*)a.y,
                           a.rstd, a.rows, a.H, a.eps);
    }
    return launch_error();
}

template <typename T, int VEC>
static hipError_t dispatch(const FwdArgs& a, bool residual, hipStream_t s) {
    Geometry g;
    if (!choose_geometry(a.H, VEC, residual, &g)) return hipErrorInvalidValue;
    // bf16 rows of 8193-16384 elements: 512 x 4 instead of 1024 x 2 (one row
    // per workgroup either way).  Measured on 4096 x 16384: forward 46.9 ->
    // 38.5 us, residual forward 92.9 -> 88.7; 512 x 8 and 512 x 16 for the
    // wider rows and 512 x 4 for fp32 were slower.
    if (sizeof(T) == 2 && VEC > 1 && g.team == 1024 && g.nch == 2) {
        g.team = 512;
        g.nch = 4;
    }

#define RMS_CASE(TM, NC) \
    if (g.team == TM && g.nch == NC) return launch_cfg<T, VEC, TM, NC>(a, residual, s);
    RMS_CASE(1, 1) RMS_CASE(2, 1) RMS_CASE(4, 1) RMS_CASE(8, 1) RMS_CASE(16, 1) RMS_CASE(32, 1)
    RMS_CASE(64, 1) RMS_CASE(64, 2) RMS_CASE(128, 2) RMS_CASE(256, 2) RMS_CASE(512, 1)
    RMS_CASE(512, 2) RMS_CASE(512, 4)
    RMS_CASE(1024, 2) RMS_CASE(1024, 4) RMS_CASE(1024, 8)
    // 1024 x 16 only where the widest row (65536) needs it: not for bf16 with
    // 128-bit access, whose 1024 x 8 tile already covers 65536.
    if constexpr (1024 * 8 * VEC < 65536) { RMS_CASE(1024, 16) }
#undef RMS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(DType dt, int vec, const FwdArgs& a, bool residual, hipStream_t s) {
    if (dt == DType::F32) {
        return vec == 4 ? dispatch<float, 4>(a, residual, s) : dispatch<float, 1>(a, residual, s);
    }
    return vec == 8 ? dispatch<bf16_t, 8>(a, residual, s) : dispatch<bf16_t, 1>(a, residual, s);
}

}  // namespace rms
