// Backward row pass for rows too wide for the register tiles of
// bwd_rows_kernel, gfx950: an LDS-staged form for 1024-lane teams with two
// 16-byte chunks per lane (the next row staged in LDS), a row-in-LDS form for
// rows of up to 128 KB of x and dy without a residual-stream gradient, and a
// streaming form for the rest.  All write the same per-workgroup dw partial
// rows as bwd_rows_kernel, reduced by the same dw reduce pass.
//
// P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）":
//   §5.3 the backward formulas; §5.4 dw in two passes rather than atomics.
#include <utility>

#include "bwd_row_math.hpp"
#include "launch.hpp"

// 1: rows of 1024-lane teams with four 16-byte chunks per lane and no
// residual-stream gradient are held in LDS (bwd_rows_ldsrow_kernel).
#ifndef RMS_BWD_LDSROW
#define RMS_BWD_LDSROW 1
#endif

namespace rms {

// Rows too wide for the register tiles (1024-lane teams with 4 or more
// chunks per lane).  Holding such a row in registers across its row sum
// spills, so a workgroup of WW lanes owns one row at a time and streams it
// twice in slices of WW * VEC elements: pass A forms the row sums, pass B reads
// each slice again (from L2 where it still holds them: pass A's loads are
// cached, pass B's are the last use) to form dx and the dw terms.  Only the
// dw column sums stay in registers (NS x VEC per lane).  The next slice's
// loads are in flight while the current one is used, also across the pass
// and row boundaries.  Rows are dealt round-robin to the G workgroups; each
// writes one partial row of dw sums, as bwd_rows_kernel does.  Workgroups
// of WW = 1024 lanes up to 4 slices; wider rows use 512 lanes, whose waves
// have twice the registers for the larger share of dw sums.

template <typename T, int VEC, int WW, int NS, bool DRES, bool RSTD>
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
    constexpr bool has_rstd = RSTD;  // saved statistic (else r from x)
    const double inv_h = 1.0 / (double)H;
    const uint32_t row_bytes = (uint32_t)H * (uint32_t)sizeof(T);
    // Slice s of a row is addressed through a resource that starts at the
    // slice and ends at the row's end, so one lane offset serves every slice
    // and lanes past H read zeros and store nothing.  The sizes are made
    // uniform explicitly (as a vector saturating subtract they would turn
    // every access into a loop over lanes).
    const int lcol = lt * VEC;
    const uint32_t loff = (uint32_t)lcol * (uint32_t)sizeof(T);
    constexpr uint32_t SLB = SL * sizeof(T);
    auto sres = [&](const T* rowp, int s, uint32_t n) {
        const uint32_t rest = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(n > s * SLB ? n - s * SLB : 0u));
        return buf_rsrc(rowp + s * SL, rest);
    };
    // w is read in both passes of every row; up to 128 KB of it is kept in
    // LDS (every build but fp32 at 65536), the rest re-read from L2.
    constexpr bool kWLds = (size_t)NS * SL * sizeof(T) <= 131072;
    __shared__ __align__(16) T wl[kWLds ? NS * SL : 1];
    if constexpr (kWLds) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            *reinterpret_cast<Pack<T, VEC>*>(&wl[s * SL + lcol]) =
                buf_load_pack<T, VEC>(sres(w, s, row_bytes), loff);
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
        q.x = buf_load_pack<T, VEC>(sres(x + off, s, n), loff);
        q.dy = buf_load_pack<T, VEC>(sres(dy + off, s, n), loff);
        if constexpr (!kWLds) q.w = buf_load_pack<T, VEC>(sres(w, s, row_bytes), loff);
    };
    auto load_b = [&](int64_t row, int s, Slice& q) {
        const int64_t off = row * (int64_t)H;
        q.x = buf_load_pack<T, VEC, kNtLoad>(sres(x + off, s, row_bytes), loff);
        q.dy = buf_load_pack<T, VEC, kNtLoad>(sres(dy + off, s, row_bytes), loff);
        if constexpr (!kWLds) q.w = buf_load_pack<T, VEC>(sres(w, s, row_bytes), loff);
        if constexpr (DRES) q.dr = buf_load_pack<T, VEC, kNtLoad>(sres(dres + off, s, row_bytes), loff);
    };

    const int64_t G = gridDim.x;
    constexpr bool kRevB = WW == 1024;  // pass B last slice first
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
            else load_b(row, kRevB ? NS - 1 : 0, buf[0]);
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
        // Pass B: dx and the dw terms, slice by slice while the next one
        // loads (after the last, the next row's first, into buffer 0).  The
        // 1024-lane builds go last slice first, so that the slices pass A read
        // last are re-read while L2 still holds them: slice s from buffer
        // (s + 1) & 1.  (Measured at bf16 2048 x 32768 with dres: 113.8 ->
        // 109.9 us.  In the 512-lane builds, rows of 256 KB, pass A's data is
        // gone either way, and the reversed order measured 0.6-3% slower.)
        T* const dxr = dx + row * (int64_t)H;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int s = kRevB ? NS - 1 - j : j;
            if (j + 1 < NS) load_b(row, kRevB ? s - 1 : s + 1, buf[kRevB ? s & 1 : (s + 1) & 1]);
            else load_a(row + G, 0, buf[0]);
            const Slice& q = buf[kRevB ? (s + 1) & 1 : s & 1];
            float xv[VEC], dyv[VEC], wc[VEC], drv[VEC], o[VEC];
            unpack(q.x, xv);
            unpack(q.dy, dyv);
            w_slice(s, q.w, wc);
            if constexpr (DRES) unpack(q.dr, drv);
            dx_chunk<T, VEC, DRES>(xv, dyv, wc, drv, kq, o, acc[s]);
            buf_store_vec<T, VEC, kNtStore, DRES>(sres(dxr, s, row_bytes), loff, o);
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
template <typename T, int VEC, bool DRES, bool RSTD>
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
    constexpr bool has_rstd = RSTD;  // saved statistic (else r from x)
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
        // The waits count this row's dx stores after the staging loads: keep
        // the compiler from moving a store above them.
        asm volatile("" ::: "memory");
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
        // When r is recomputed, the row is unpacked again below and only the
        // packed row stays live across the row sums: kept from pass A, its
        // floats and the fp64 squares' operands spilled at 128 VGPRs (scratch
        // accesses would also upset the counted waits).  With a saved rstd
        // they fit, and keeping them measured 3% faster.
        if constexpr (!RSTD) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                opaque(px[c]);
                opaque(pdy[c]);
            }
        }
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

// LDS byte address of a __shared__ object (device pass only).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
#else
    (void)p;
    return 0u;
#endif
}

// Two 16-byte LDS reads at a + OFF and b + OFF with their lgkmcnt wait, in
// one asm statement.  Read as ordinary LDS loads, regions that direct loads
// fill make the compiler wait first for every direct load in flight (it
// cannot tell the regions apart), which would drain the loads of the chunks
// still to come.
template <int OFF>
__device__ __forceinline__ void lds_read2(uint32_t a, uint32_t b, u32x4& va, u32x4& vb) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile(
        "ds_read_b128 %0, %2 offset:%4\n\t"
        "ds_read_b128 %1, %3 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(va), "=&v"(vb)
        : "v"(a), "v"(b), "i"(OFF)
        : "memory");
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Rows of 16385-32768 bf16 or 8193-16384 fp32 elements (WG lanes with NCH
// 16-byte chunks each, 512 x 8), without a residual-stream gradient: one row
// at a time, its x and dy held in LDS (128 KB), so that pass B reads them from
// LDS instead of again from the caches.  Each wave stages its lanes' part of
// every chunk in its own LDS region with direct buffer-to-LDS loads; pass A
// waits for each chunk as it is summed, and pass B, after reading chunk c
// back, refills that region with chunk c of the workgroup's next row.  w
// stays in registers (512 lanes leave room for it beside the dw sums).
// Chunk c of a row is addressed through a resource that starts at the chunk
// and ends at the row's end, so one lane offset serves every chunk and lanes
// past H read zeros.  The compiler does not order an LDS read after the
// direct load that fills it, so the waits are explicit; vmcnt counts the
// loads, direct loads and stores of a wave in issue order:
//   * the first row and w are waited for in full before the loop (so the
//     compiler, too, knows that w has landed and adds no wait for it);
//   * a later row's chunk c was staged in the previous row's pass B, which
//     issues per chunk its two loads and then its dx store: 1 + 3 (NCH - 1 - c)
//     operations are younger.
template <int NCH, int C>
__device__ __forceinline__ void wait_chunk() {
    __builtin_amdgcn_s_waitcnt(wait_vm(1 + 3 * (NCH - 1 - C)));
    asm volatile("" ::: "memory");
}

template <typename T, int VEC, int WG, int NCH, bool RSTD>
__global__ __launch_bounds__(WG) void bwd_rows_ldsrow_kernel(
    const T* dy, const T* __restrict__ x, const T* __restrict__ w,
    const float* __restrict__ rstd, T* dx, float* __restrict__ partial, int64_t rows, int H,
    int ldp, float eps) {
    constexpr int NWT = WG / kWave;
    static_assert(3 * NCH <= 63, "vmcnt range");
    constexpr bool kNtLoad = RMS_BWD_NT_LOAD != 0;
    constexpr bool kNtStore = RMS_BWD_NT_STORE != 0;
    constexpr int aux = kNtLoad ? kAuxNt : 0;
    constexpr int kChunkElems = WG * VEC;               // elements per chunk
    constexpr uint32_t kChunkBytes = kChunkElems * sizeof(T);
    constexpr uint32_t kLdsChunk = WG * 16;             // LDS bytes per chunk
    __shared__ double red[2 * 2 * NWT];
    __shared__ __align__(16) u32x4 stage[2][NCH][WG];  // x, dy of the current row

    const int lt = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(lt / kWave);
    constexpr bool has_rstd = RSTD;  // saved statistic (else r from x)
    const double inv_h = 1.0 / (double)H;
    const uint32_t row_bytes = (uint32_t)H * (uint32_t)sizeof(T);
    const uint32_t loff = (uint32_t)lt * VEC * (uint32_t)sizeof(T);  // lane offset in a chunk
    // Bytes of the row from chunk c on (0 past the row).  Uniform, and kept
    // in scalar registers: formed as a vector saturating subtract, a
    // resource size would make the compiler loop over lanes at every load.
    auto rest = [&](int c, uint32_t n) {
        return (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(n > c * kChunkBytes ? n - c * kChunkBytes : 0u));
    };
    Pack<T, VEC> wp[NCH];
    static_for<NCH>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        wp[c] = buf_load_pack<T, VEC>(buf_rsrc(w + c * kChunkElems, rest(c, row_bytes)), loff);
    });
    float acc[NCH][VEC];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
    }
    // Chunk c of row `row` (past the end: empty resources, nothing is read):
    // two direct loads.
    auto stage_chunk = [&](int64_t row, int c) {
        const bool ok = row < rows;
        const int64_t off = (ok ? row * (int64_t)H : 0) + c * kChunkElems;
        const uint32_t n = ok ? rest(c, row_bytes) : 0u;
        buf_load_lds16<aux>(buf_rsrc(x + off, n), &stage[0][c][wave * kWave], loff);
        buf_load_lds16<aux>(buf_rsrc(dy + off, n), &stage[1][c][wave * kWave], loff);
    };
    auto load_rs = [&](int64_t row) {
        const BufRes rr = (has_rstd && row < rows) ? buf_rsrc(rstd + row, 4u) : buf_rsrc(x, 0u);
        return buf_load_f32(rr, 0u);
    };
    const uint32_t ax = lds_addr(&stage[0][0][lt]);
    const uint32_t ady = lds_addr(&stage[1][0][lt]);
    // Chunk c as read back; lanes past H get zeros (the region may hold an
    // earlier row's bytes there).
    auto read_chunk = [&](auto cc, Pack<T, VEC>& px, Pack<T, VEC>& pdy) {
        constexpr int c = decltype(cc)::value;
        lds_read2<c * kLdsChunk>(ax, ady, px.v, pdy.v);
        if (loff + c * kChunkBytes >= row_bytes) {
            px = zero_pack<T, VEC>();
            pdy = zero_pack<T, VEC>();
        }
    };

    const int64_t G = gridDim.x;
    int64_t row = blockIdx.x;
    float rs = load_rs(row);
    for (int c = 0; c < NCH; ++c) stage_chunk(row, c);
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    asm volatile("" ::: "memory");
    int set = 0;
    for (; row < rows; row += G, set ^= 1) {
        // w stays packed between rows: an empty asm that "changes" it keeps
        // the compiler from hoisting its unpacked floats out of the loop.
#pragma unroll
        for (int c = 0; c < NCH; ++c) asm volatile("" : "+v"(wp[c].v));
        // Pass A: the row sums, each chunk as soon as it has landed.
        double cs = 0.0, ss = 0.0;
        static_for<NCH>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            wait_chunk<NCH, c>();
            Pack<T, VEC> px, pdy;
            read_chunk(cc, px, pdy);
            float xv[VEC], dyv[VEC], wc[VEC];
            unpack(px, xv);
            unpack(pdy, dyv);
            unpack(wp[c], wc);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                cs += prod3_64(wc[k], dyv[k], xv[k], (T*)nullptr);
                if (!has_rstd) ss += sq64(xv[k], (T*)nullptr);
            }
        });
        double* slots = red + set * 2 * NWT;
        cs = team_sum_nofence<WG>(cs, slots);
        double r;
        if (has_rstd) {
            r = (double)rs;
        } else {
            ss = team_sum_nofence<WG>(ss, slots + NWT);
            r = rsqrt_f64(ss * inv_h + (double)eps);
        }
        const RowK kq = row_k(r, cs, inv_h, true);
        rs = load_rs(row + G);
        asm volatile("" ::: "memory");  // rstd's load stays older than the chunks' loads
        // Pass B: dx and the dw terms from the chunks in LDS; each chunk's
        // region is refilled with the next row's chunk once read.
        T* const dxr = dx + row * (int64_t)H;
        static_for<NCH>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            Pack<T, VEC> px, pdy;
            read_chunk(cc, px, pdy);
            stage_chunk(row + G, c);
            // The waits count this chunk's dx store after its two loads: keep
            // the compiler from moving the store (or anything) above them.
            asm volatile("" ::: "memory");
            float xv[VEC], dyv[VEC], wc[VEC], drv[VEC], o[VEC];
            unpack(px, xv);
            unpack(pdy, dyv);
            unpack(wp[c], wc);
            dx_chunk<T, VEC, false>(xv, dyv, wc, drv, kq, o, acc[c]);
            buf_store_vec<T, VEC, kNtStore>(buf_rsrc(dxr + c * kChunkElems, rest(c, row_bytes)),
                                            loff, o);
        });
    }
    // The chunks staged past the workgroup's last row read nothing but still
    // write LDS: wait for them before the workgroup can end.
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    float* prow = partial + (int64_t)blockIdx.x * ldp;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int col = c * kChunkElems + lt * VEC;
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
    auto go = [&](auto dres_c, auto rstd_c) {
        constexpr bool D = decltype(dres_c)::value, RS = decltype(rstd_c)::value;
        RMS_LAUNCH((bwd_rows_wide_kernel<T, VEC, WW, NS, D, RS>), dim3(a.G), dim3(WW), 0, s,
                           (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd,
                           (const T*)a.dres, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    };
    bwd_variant(a, go);
    return launch_error();
}

template <typename T, int VEC>
static hipError_t launch_rows_wide(const BwdArgs& a, hipStream_t s) {
    const int64_t n1024 = (a.H + 1024 * VEC - 1) / (1024 * VEC);
    if constexpr (VEC > 1 && RMS_BWD_LDSROW) {
        if (n1024 <= 4 && !a.dres) {
            if (a.rstd) {
                RMS_LAUNCH((bwd_rows_ldsrow_kernel<T, VEC, 512, 8, true>), dim3(a.G),
                                   dim3(512), 0, s, (const T*)a.dy, (const T*)a.x, (const T*)a.w,
                                   a.rstd, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
            } else {
                RMS_LAUNCH((bwd_rows_ldsrow_kernel<T, VEC, 512, 8, false>), dim3(a.G),
                                   dim3(512), 0, s, (const T*)a.dy, (const T*)a.x, (const T*)a.w,
                                   a.rstd, (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
            }
            return launch_error();
        }
    }
    if (n1024 <= 4) return launch_wide_cfg<T, VEC, 1024, 4>(a, s);
    const int64_t n512 = (a.H + 512 * VEC - 1) / (512 * VEC);
    if (n512 <= 16) return launch_wide_cfg<T, VEC, 512, 16>(a, s);
    // 32 slices of 512 x VEC only where RMSNORM_MAX_H (65536) needs them: not
    // for bf16 with 128-bit access (16 slices reach 65536), so that build is
    // not instantiated.
    if constexpr (512 * 16 * VEC < 65536) {
        if (n512 <= 32) return launch_wide_cfg<T, VEC, 512, 32>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename T, int VEC>
static hipError_t launch_rows_staged(const BwdArgs& a, hipStream_t s) {
    auto go = [&](auto dres_c, auto rstd_c) {
        constexpr bool D = decltype(dres_c)::value, RS = decltype(rstd_c)::value;
        RMS_LAUNCH((bwd_rows_staged_kernel<T, VEC, D, RS>), dim3(a.G), dim3(1024), 0, s,
                           (const T*)a.dy, (const T*)a.x, (const T*)a.w, a.rstd, (const T*)a.dres,
                           (T*)a.dx, a.partial, a.rows, a.H, a.ldp, a.eps);
    };
    bwd_variant(a, go);
    return launch_error();
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
