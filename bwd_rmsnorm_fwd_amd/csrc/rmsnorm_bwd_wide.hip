// Backward row pass for rows too wide for the register tiles of
// bwd_rows_kernel, gfx950: an LDS-staged form for 1024-lane teams with two
// 16-byte chunks per lane, and a streaming form for wider rows.  Both write
// the same per-workgroup dw partial rows as bwd_rows_kernel, reduced by the
// same dw reduce pass.
//
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）":
//   §5.3 the backward formulas; §5.4 dw in two passes rather than atomics.
#include "bwd_row_math.hpp"
#include "launch.hpp"

namespace rms {

// Rows too wide for the register tiles (1024-lane teams with 4 or more
// chunks per lane).  Holding such a row in registers across its row sum
// spills, so a workgroup of WW lanes owns one row at a time and streams it
// twice in slices of WW * VEC elements: pass A forms the row sums, pass B reads
// each slice again (from L2 or the Infinity Cache: pass A's loads are
// cached, pass B's are the last use) to form dx and the dw terms.  Only the
// dw column sums stay in registers (NS x VEC per lane).  The next slice's
// loads are in flight while the current one is used, also across the pass
// and row boundaries.  Rows are dealt round-robin to the G workgroups; each
// writes one partial row of dw sums, as bwd_rows_kernel does.  Workgroups
// of WW = 1024 lanes up to 4 slices; wider rows use 512 lanes, whose waves
// have twice the registers for the larger share of dw sums.

template <typename T, int VEC, int WW, int NS, bool DRES>
__global__ __launch_bounds__(WW) void bwd_rows_wide_kernel(
    const T* dy, const T* __restrict__ x, const T* __restrict__ w,
    const float* __restrict__ rstd, const T* dres, T* dx, float* __restrict__ partial,
    int64_t rows, int H, int ldp, float eps) {
    static_assert(NS >= 2 && (NS & (NS - 1)) == 0, "NS: a power of two, at least 2");
    constexpr int NWT = WW / kWave;
    constexpr int SL = WW * VEC;  // elements per slice
    constexpr bool kNtLoad = DRES ? RMS_DRES_NT_LOAD != 0 : RMS_BWD_NT_LOAD != 0;
    constexpr bool kNtStore = DRES ? RMS_DRES_NT_STORE != 0 : RMS_BWD_NT_STORE != 0;
    // Two slot sets used by alternate rows, each for c and sum x^2.
    __shared__ double red[2 * 2 * NWT];

    const int lt = threadIdx.x;
    const bool has_rstd = rstd != nullptr;
    const double inv_h = 1.0 / (double)H;
    const uint32_t row_bytes = (uint32_t)H * (uint32_t)sizeof(T);
    // The lane's offset in slice s; chunks past H (and slices past the row)
    // read zeros and are not stored.  Formed when used rather than kept: the
    // registers go to the dw sums.
    const int lcol = lt * VEC;
    auto voff = [&](int s) -> uint32_t {
        const int col = s * SL + lcol;
        return col < H ? (uint32_t)col * (uint32_t)sizeof(T) : kBufOutside;
    };
    const BufRes rw = buf_rsrc(w, row_bytes);
    // w is read in both passes of every row; up to 128 KB of it is kept in
    // LDS (every build but fp32 at 65536), the rest re-read from L2.
    constexpr bool kWLds = (size_t)NS * SL * sizeof(T) <= 131072;
    __shared__ __align__(16) T wl[kWLds ? NS * SL : 1];
    if constexpr (kWLds) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            *reinterpret_cast<Pack<T, VEC>*>(&wl[s * SL + lcol]) = buf_load_pack<T, VEC>(rw, voff(s));
        }
        __syncthreads();
    }
    auto w_slice = [&](int s, const Pack<T, VEC>& qw, float (&wc)[VEC]) {
        if constexpr (kWLds) unpack(*reinterpret_cast<const Pack<T, VEC>*>(&wl[s * SL + lcol]), wc);
        else unpack(qw, wc);
    };
    float acc[NS][VEC];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[s][k] = 0.f;
    }

    struct Slice {
        Pack<T, VEC> x, dy, w, dr;
    };
    // Pass A's loads: row `row` if it exists (else an empty resource: the
    // loads return zeros and read nothing), cached for pass B.
    auto load_a = [&](int64_t row, int s, Slice& q) {
        const bool ok = row < rows;
        const int64_t off = ok ? row * (int64_t)H : 0;
        const uint32_t n = ok ? row_bytes : 0u;
        q.x = buf_load_pack<T, VEC>(buf_rsrc(x + off, n), voff(s));
        q.dy = buf_load_pack<T, VEC>(buf_rsrc(dy + off, n), voff(s));
        if constexpr (!kWLds) q.w = buf_load_pack<T, VEC>(rw, voff(s));
    };
    auto load_b = [&](int64_t row, int s, Slice& q) {
        const int64_t off = row * (int64_t)H;
        q.x = buf_load_pack<T, VEC, kNtLoad>(buf_rsrc(x + off, row_bytes), voff(s));
        q.dy = buf_load_pack<T, VEC, kNtLoad>(buf_rsrc(dy + off, row_bytes), voff(s));
        if constexpr (!kWLds) q.w = buf_load_pack<T, VEC>(rw, voff(s));
        if constexpr (DRES) q.dr = buf_load_pack<T, VEC, kNtLoad>(buf_rsrc(dres + off, row_bytes), voff(s));
    };

    const int64_t G = gridDim.x;
    Slice buf[2];
    int set = 0;
    int64_t row = blockIdx.x;
    load_a(row, 0, buf[0]);
    for (; row < rows; row += G, set ^= 1) {
        // Pass A: the row sums, slice s while slice s + 1 loads (after the
        // last slice, pass B's first).
        double cs = 0.0, ss = 0.0;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) load_a(row, s + 1, buf[(s + 1) & 1]);
            else load_b(row, 0, buf[0]);
            const Slice& q = buf[s & 1];
            float xv[VEC], dyv[VEC], wc[VEC];
            unpack(q.x, xv);
            unpack(q.dy, dyv);
            w_slice(s, q.w, wc);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                cs += prod3_64(wc[k], dyv[k], xv[k], (T*)nullptr);
                if (!has_rstd) ss += sq64(xv[k], (T*)nullptr);
            }
            // Keep the schedule one slice ahead: without this fence the
            // unrolled slices' loads are hoisted together and spill.
            __builtin_amdgcn_sched_barrier(0);
        }
        double* slots = red + set * 2 * NWT;
        cs = team_sum_alt<WW>(cs, slots);
        double r;
        if (has_rstd) {
            r = (double)rstd[row];
        } else {
            ss = team_sum_alt<WW>(ss, slots + NWT);
            r = rsqrt_f64(ss * inv_h + (double)eps);
        }
        const RowK kq = row_k(r, cs, inv_h, true);
        // Pass B: dx and the dw terms, slice s while slice s + 1 loads
        // (after the last slice, the next row's first).
        const BufRes rdx = buf_rsrc(dx + row * (int64_t)H, row_bytes);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) load_b(row, s + 1, buf[(s + 1) & 1]);
            else load_a(row + G, 0, buf[0]);
            const Slice& q = buf[s & 1];
            float xv[VEC], dyv[VEC], wc[VEC], drv[VEC], o[VEC];
            unpack(q.x, xv);
            unpack(q.dy, dyv);
            w_slice(s, q.w, wc);
            if constexpr (DRES) unpack(q.dr, drv);
            dx_chunk<T, VEC, DRES>(xv, dyv, wc, drv, kq, o, acc[s]);
            buf_store_vec<T, VEC, kNtStore, DRES>(rdx, voff(s), o);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // The workgroup's partial row (zeros if it had no rows).
    float* prow = partial + (int64_t)blockIdx.x * ldp;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int col = s * SL + lt * VEC;
        if (col < H) {
            if constexpr (VEC == 1) {
                prow[col] = acc[s][0];
            } else {
#pragma unroll
                for (int k = 0; k < VEC; k += 4) {
                    u32x4 v;
                    v.x = __float_as_uint(acc[s][k]);
                    v.y = __float_as_uint(acc[s][k + 1]);
                    v.z = __float_as_uint(acc[s][k + 2]);
                    v.w = __float_as_uint(acc[s][k + 3]);
                    st128<false>(prow + col + k, v);
                }
            }
        }
    }
}

// 1024-lane teams with two 16-byte chunks per lane (8193-16384 bf16 or
// 4097-8192 fp32 elements): the row and a prefetched successor do not both
// fit in registers, so each wave stages its lanes' part of the next row in
// its own region of LDS with direct buffer-to-LDS loads while it finishes
// the current row from registers.  The compiler does not order an LDS read
// after the direct load that fills it, so the waits are explicit: before a
// row is read from LDS, every memory operation older than the previous
// row's dx stores has completed (vmcnt), and the LDS reads have returned
// (lgkmcnt) before the region is refilled.
template <typename T, int VEC, bool DRES>
__global__ __launch_bounds__(1024) void bwd_rows_staged_kernel(
    const T* dy, const T* __restrict__ x, const T* __restrict__ w,
    const float* __restrict__ rstd, const T* dres, T* dx, float* __restrict__ partial,
    int64_t rows, int H, int ldp, float eps) {
    constexpr int TEAM = 1024, NCH = 2, NWT = TEAM / kWave;
    constexpr int NT = DRES ? 3 : 2;  // row tensors staged: x, dy (, dres)
    constexpr bool kNtLoad = DRES ? RMS_DRES_NT_LOAD != 0 : RMS_BWD_NT_LOAD != 0;
    constexpr bool kNtStore = DRES ? RMS_DRES_NT_STORE != 0 : RMS_BWD_NT_STORE != 0;
    constexpr int aux = kNtLoad ? kAuxNt : 0;
    __shared__ double red[2 * 2 * NWT];
    __shared__ __align__(16) u32x4 stage[NT][NCH][TEAM];
    __shared__ __align__(16) u32x4 wst[NCH][TEAM];  // w, read from LDS in the loop

    const int lt = threadIdx.x;
    const int wave = lt / kWave;
    const bool has_rstd = rstd != nullptr;
    const double inv_h = 1.0 / (double)H;
    const uint32_t row_bytes = (uint32_t)H * (uint32_t)sizeof(T);
    uint32_t voff[NCH];
    bool cok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * TEAM + lt) * VEC;
        cok[c] = col < H;
        voff[c] = cok[c] ? (uint32_t)col * (uint32_t)sizeof(T) : kBufOutside;
    }
    float acc[NCH][VEC];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
    }
    // w goes to LDS once, so that no global load in the loop is younger than
    // the staged row (a wait for it would wait for the staging too).
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * TEAM + lt) * VEC;
        wst[c][lt] = cok[c] ? ld128<false>(w + col) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    auto weights = [&](int c, float (&wc)[VEC]) {
        Pack<T, VEC> p;
        p.v = wst[c][lt];
        unpack(p, wc);
    };
    auto lds = [&](int t, int c) { return (void*)&stage[t][c][wave * kWave]; };
    // Stage row `row` (an empty resource past the end: nothing is read) and
    // load its rstd; always the same NT * NCH + 1 memory operations.
    auto stage_row = [&](int64_t row, float& rs) {
        const bool ok = row < rows;
        const int64_t off = ok ? row * (int64_t)H : 0;
        const uint32_t n = ok ? row_bytes : 0u;
        const BufRes rx = buf_rsrc(x + off, n);
        const BufRes rdy = buf_rsrc(dy + off, n);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            buf_load_lds16<aux>(rx, lds(0, c), voff[c]);
            buf_load_lds16<aux>(rdy, lds(1, c), voff[c]);
            if constexpr (DRES) buf_load_lds16<aux>(buf_rsrc(dres + off, n), lds(2, c), voff[c]);
        }
        const BufRes rr = (has_rstd && ok) ? buf_rsrc(rstd + row, 4u) : buf_rsrc(x, 0u);
        rs = buf_load_f32(rr, 0u);
    };

    const int64_t G = gridDim.x;
    int64_t row = blockIdx.x;
    float rs_next;
    stage_row(row, rs_next);
    int set = 0;
    bool first = true;
    for (; row < rows; row += G, set ^= 1) {
        if (first) __builtin_amdgcn_s_waitcnt(wait_vm(0));
        else __builtin_amdgcn_s_waitcnt(wait_vm(NCH));
        first = false;
        Pack<T, VEC> px[NCH], pdy[NCH], pdr[DRES ? NCH : 1];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            px[c].v = stage[0][c][lt];
            pdy[c].v = stage[1][c][lt];
            if constexpr (DRES) pdr[c].v = stage[2][c][lt];
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        const float rs = rs_next;
        stage_row(row + G, rs_next);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (!cok[c]) {
                px[c] = zero_pack<T, VEC>();
                pdy[c] = zero_pack<T, VEC>();
                if constexpr (DRES) pdr[c] = zero_pack<T, VEC>();
            }
        }
        double cs = 0.0, ss = 0.0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float xv[VEC], dyv[VEC], wc[VEC];
            unpack(px[c], xv);
            unpack(pdy[c], dyv);
            weights(c, wc);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                cs += prod3_64(wc[k], dyv[k], xv[k], (T*)nullptr);
                if (!has_rstd) ss += sq64(xv[k], (T*)nullptr);
            }
        }
        double* slots = red + set * 2 * NWT;
        cs = team_sum_nofence<1024>(cs, slots);
        double r;
        if (has_rstd) {
            r = (double)rs;
        } else {
            ss = team_sum_nofence<1024>(ss, slots + NWT);
            r = rsqrt_f64(ss * inv_h + (double)eps);
        }
        const RowK kq = row_k(r, cs, inv_h, true);
        const BufRes rdx = buf_rsrc(dx + row * (int64_t)H, row_bytes);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float xv[VEC], dyv[VEC], wc[VEC], drv[VEC], o[VEC];
            unpack(px[c], xv);
            unpack(pdy[c], dyv);
            weights(c, wc);
            if constexpr (DRES) unpack(pdr[c], drv);
            dx_chunk<T, VEC, DRES>(xv, dyv, wc, drv, kq, o, acc[c]);
            buf_store_vec<T, VEC, kNtStore, DRES>(rdx, voff[c], o);
        }
    }
    // The loads staged past the workgroup's last row read nothing (their
    // resources are empty), but they still write LDS: wait for them before
    // the workgroup can end and its LDS go to another.
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    float* prow = partial + (int64_t)blockIdx.x * ldp;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = (c * TEAM + lt) * VEC;
        if (col < H) {
#pragma unroll
            for (int k = 0; k < VEC; k += 4) {
                u32x4 v;
                v.x = __float_as_uint(acc[c][k]);
                v.y = __float_as_uint(acc[c][k + 1]);
                v.z = __float_as_uint(acc[c][k + 2]);
                v.w = __float_as_uint(acc[c][k + 3]);
                st128<false>(prow + col + k, v);
            }
        }
    }
}

// Rows the geometry table gives a 1024-lane team with 4 or more chunks per
// lane (wider than 16384 bf16 or 8192 fp32 elements with 128-bit access,
// 2048 with scalar access): the streaming kernel, in 1024-lane workgroups
// when the row takes at most 4 slices of them, else in 512-lane workgroups,
// with the smallest power-of-two slice count that covers the row.  Measured against the register tiles: bf16 2048 x 32768 row pass 135.6
// -> 97.5 us, 1024 x 65536 340.5 -> 129.6, 2048 x 32768 with dres 242.5 ->
// 115.1; at 4096 x 16384 the 1024 x 2 tile stays (84.5 vs 94.0).
template <typename T, int VEC, int WW, int NS>
static hipError_t launch_wide_cfg(const BwdArgs& a, hipStream_t s) {
    if (a.dres) {
        hipLaunchKernelGGL((bwd_rows_wide_kernel<T, VEC, WW, NS, true>), dim3(a.G), dim3(WW), 0, s,
                           (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd,
                           (const T*)a.dres, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    } else {
        hipLaunchKernelGGL((bwd_rows_wide_kernel<T, VEC, WW, NS, false>), dim3(a.G), dim3(WW), 0, s,
                           (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd,
                           (const T*)nullptr, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    }
    return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t launch_rows_wide(const BwdArgs& a, hipStream_t s) {
    const int64_t n1024 = (a.H + 1024 * VEC - 1) / (1024 * VEC);
    if (n1024 <= 4) return launch_wide_cfg<T, VEC, 1024, 4>(a, s);
    const int64_t n512 = (a.H + 512 * VEC - 1) / (512 * VEC);
    if (n512 <= 16) return launch_wide_cfg<T, VEC, 512, 16>(a, s);
    if (n512 <= 32) return launch_wide_cfg<T, VEC, 512, 32>(a, s);
    return hipErrorInvalidValue;
}

template <typename T, int VEC>
static hipError_t launch_rows_staged(const BwdArgs& a, hipStream_t s) {
    if (a.dres) {
        hipLaunchKernelGGL((bwd_rows_staged_kernel<T, VEC, true>), dim3(a.G), dim3(1024), 0, s,
                           (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd, (const T*)a.dres,
                           (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    } else {
        hipLaunchKernelGGL((bwd_rows_staged_kernel<T, VEC, false>), dim3(a.G), dim3(1024), 0, s,
                           (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd, (const T*)nullptr,
                           (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_wide(DType dt, int vec, const BwdArgs& a, hipStream_t s) {
    if (dt == DType::F32) {
        return vec == 4 ? launch_rows_wide<float, 4>(a, s) : launch_rows_wide<float, 1>(a, s);
    }
    return vec == 8 ? launch_rows_wide<bf16_t, 8>(a, s) : launch_rows_wide<bf16_t, 1>(a, s);
}

hipError_t launch_bwd_staged(DType dt, int vec, const BwdArgs& a, hipStream_t s) {
    if (dt == DType::F32) return vec == 4 ? launch_rows_staged<float, 4>(a, s) : hipErrorInvalidValue;
    return vec == 8 ? launch_rows_staged<bf16_t, 8>(a, s) : hipErrorInvalidValue;
}

}  // namespace rms
