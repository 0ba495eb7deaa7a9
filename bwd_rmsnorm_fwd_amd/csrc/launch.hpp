// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Arguments are validated by the caller; these functions only pick a
// kernel instance and launch it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <typeinfo>

namespace rms {

// Dry run (rmsnorm_set_dry_run): while active on the calling host thread,
// RMS_LAUNCH records the kernel it would launch, with its grid and block,
// instead of launching it.
bool dry_run_active();
void dry_run_record(const char* pretty, dim3 grid, dim3 block);

// A kernel instance's mangled name, carried by the type name of a constant
// that holds its address (the dry run demangles it).
template <auto K>
const char* kernel_pretty() {
    return typeid(std::integral_constant<decltype(K), K>).name();
}

#define RMS_LAUNCH(KERNEL, GRID, BLOCK, SHM, STREAM, ...)                          \
    do {                                                                         \
        if (::rms::dry_run_active())                                             \
            ::rms::dry_run_record(::rms::kernel_pretty<&KERNEL>(), GRID, BLOCK); \
        else                                                                     \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHM, STREAM, __VA_ARGS__);   \
    } while (0)

// The error of the last launch: hipGetLastError(), or success during a dry
// run, which launches nothing.
inline hipError_t launch_error() { return dry_run_active() ? hipSuccess : hipGetLastError(); }

enum class DType { F32 = 0, BF16 = 1 };

// Geometry chosen for a row width: a team of `team` lanes handles one row,
// each lane holds `nch` chunks of `vec` elements.  Each kernel sizes its
// workgroups from the geometry itself.
struct Geometry {
    int vec;
    int team;
    int nch;
};

// Returns false when H needs more than the largest register tile.
// `wide` selects the tile for the kinds that stream more row tensors (the
// residual forward, the backward with a residual-stream gradient): one
// 16-byte chunk per lane on a 512-lane team where the others use two chunks
// on 256 lanes.
bool choose_geometry(int64_t H, int vec, bool wide, Geometry* g);

// Largest vector width usable for these pointers and H (elements; 16 bytes
// worth when everything is aligned, else 1).
int choose_vec(DType dt, int64_t H, const void* const* ptrs, int nptrs);

struct FwdArgs {
    const void* x;
    const void* res;  // residual variant only
    const void* w;
    void* h;          // residual variant only
    void* y;
    float* rstd;      // may be null
    int64_t rows;
    int H;
    float eps;
};

struct BwdArgs {
    const void* dy;
    const void* x;
    const void* w;
    const float* rstd;  // null: recompute
    const void* dres;   // may be null
    void* dx;
    float* partial;     // [G][ldp] fp32
    int64_t rows;
    int H;
    int ldp;            // partial row stride (floats)
    int G;              // workgroups of the row pass
    float eps;
};

// Number of workgroups of the backward row pass and the partial row stride.
// Pure functions of (rows, H, dtype, vec): the reduction order, and so the
// bits of dw, depend on nothing else.
int bwd_groups(int64_t rows, int64_t H, DType dt);
int partial_ld(int64_t H);

hipError_t launch_fwd(DType dt, int vec, const FwdArgs& a, bool residual, hipStream_t s);
hipError_t launch_bwd_rows(DType dt, int vec, const BwdArgs& a, hipStream_t s);
// Rows of 1024-lane teams: with two 16-byte chunks per lane (vec > 1), the
// LDS-staged kernel; with four or more, the row-in-LDS kernel where x and dy
// of a row fit in LDS and no dres is given (launch_bwd_wide picks it), else
// the streaming kernel.
hipError_t launch_bwd_staged(DType dt, int vec, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_wide(DType dt, int vec, const BwdArgs& a, hipStream_t s);
hipError_t launch_dw_reduce(DType dt, const float* partial, int G, int ldp, int H, void* dw,
                            hipStream_t s);
hipError_t launch_splitrow(DType dt, int vec, const FwdArgs& a, float* partials, int splits,
                           hipStream_t s);

struct GemvArgs {
    const void* A;    // [N][K]
    const void* x;    // [K]
    void* y;          // [N]
    float* partials;  // [splits][N] (unused when splits == 1)
    int N;
    int K;
    int seg;          // segment length (multiple of the vector width)
    int splits;
    int team;         // lanes per row (power of two, <= 64)
};

hipError_t launch_gemv(DType dt, int vec, const GemvArgs& a, hipStream_t s);

}  // namespace rms
