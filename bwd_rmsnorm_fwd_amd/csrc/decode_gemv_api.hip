// C ABI of the split-K decode matrix-vector product (include/decode_gemv.h):
// validation, vector width and team selection, launch.  No allocation.
#include <stdint.h>

#include "../../include/decode_gemv.h"
#include "launch.hpp"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

size_t decode_gemv_partials_count(int64_t N, int splits) {
    if (N < 1 || splits < 1 || splits > DECODE_GEMV_MAX_SPLITS) return 0;
    return splits == 1 ? 0 : (size_t)N * (size_t)splits;
}

rmsnorm_status_t decode_gemv_splitk(const void* A, const void* x, void* y, float* partials,
                                    size_t partials_count, int64_t N, int64_t K, int splits,
                                    rmsnorm_dtype_t dtype, hipStream_t stream) {
    if (dtype != RMSNORM_F32 && dtype != RMSNORM_BF16) return RMSNORM_EINVAL;
    if (N < 1 || K < 1 || N > INT32_MAX || K > INT32_MAX) return RMSNORM_EINVAL;
    if (splits < 1 || splits > DECODE_GEMV_MAX_SPLITS) return RMSNORM_EINVAL;
    if (!A || !x || !y) return RMSNORM_EINVAL;
    if (splits > 1 && (!partials || partials_count < (size_t)N * (size_t)splits))
        return RMSNORM_EWORKSPACE;
    const size_t e = dtype == RMSNORM_F32 ? 4 : 2;
    if (!aligned(A, e) || !aligned(x, e) || !aligned(y, e) || (partials && !aligned(partials, 4)))
        return RMSNORM_EALIGN;
    const rms::DType dt = dtype == RMSNORM_F32 ? rms::DType::F32 : rms::DType::BF16;
    const void* ptrs[2] = {A, x};
    const int vec = rms::choose_vec(dt, K, ptrs, 2);
    const int64_t nv = (K + vec - 1) / vec;                 // vectors per row
    const int64_t sv = (nv + splits - 1) / splits;          // vectors per segment
    int team = 1;
    while (team < sv && team < 64) team *= 2;
    rms::GemvArgs a{A, x, y, partials, (int)N, (int)K, (int)(sv * vec), splits, team};
    const hipError_t err = rms::launch_gemv(dt, vec, a, stream);
    return err == hipSuccess || rms::dry_run_active() ? RMSNORM_OK : RMSNORM_ELAUNCH;
}

}  // extern "C"
