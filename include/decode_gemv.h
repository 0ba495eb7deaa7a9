/*
 * decode_gemv.h -- split-K matrix-vector product for decode-sized inputs, in
 * the same library as rmsnorm.h (librmsnorm_mi355x.so).
 *
 *   y[n] = sum_k A[n][k] * x[k]        A [N][K] row-major, x [K], y [N]
 *
 * Source: the trdm.cn write-up of hand-written Triton decode kernels
 * (www.trdm.cn/news/483216), §3.1 (at batch 1 every projection is a
 * matrix-vector product; cutting the reduction dimension K into SPLIT_K
 * segments reduced in parallel into an fp32 partial buffer, then merged by a
 * separate splitk_reduce kernel, keeps the GPU busy; its q_proj is 896 ->
 * 1024), §3.3 (fp32 partials, fixed-order merge rather than atomics), §5.1
 * (the merge must not read past the split count).
 *
 * Conventions are those of rmsnorm.h: caller-owned device memory, no
 * allocation or host synchronisation, work enqueued on `stream`, status codes
 * only, bitwise-reproducible results for a given shape, dtype and split count.
 * Products are formed exactly (fp32 for bf16 inputs, fp64 for fp32 inputs) and
 * accumulated in fp64 within a segment; each segment's sum is stored as an
 * fp32 partial (as the source prescribes), and the merge adds the partials in
 * index order in fp64 and rounds once to the output dtype.
 */
#ifndef DECODE_GEMV_MI355X_H
#define DECODE_GEMV_MI355X_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest split count. */
#define DECODE_GEMV_MAX_SPLITS 64

/* Floats of partial sums decode_gemv_splitk needs: N * splits for splits > 1,
 * 0 for splits == 1; 0 for invalid arguments. */
size_t decode_gemv_partials_count(int64_t N, int splits);

/* y = A x with the reduction dimension split in `splits` segments.
 *   A         [N][K] dtype, device, read (streamed once)
 *   x         [K]    dtype, device, read
 *   y         [N]    dtype, device, written
 *   partials  fp32, device, >= decode_gemv_partials_count(N, splits) floats
 *             (may be NULL when splits == 1), scratch
 *   1 <= N, K <= 2^31 - 1; 1 <= splits <= DECODE_GEMV_MAX_SPLITS.
 * splits == 1 is one launch writing y directly; splits > 1 is the partial
 * pass followed by the splitk_reduce pass on the same stream.
 * Returns RMSNORM_EINVAL, RMSNORM_EALIGN, RMSNORM_EWORKSPACE or
 * RMSNORM_ELAUNCH as described in rmsnorm.h. */
rmsnorm_status_t decode_gemv_splitk(const void *A, const void *x, void *y, float *partials,
                                    size_t partials_count, int64_t N, int64_t K, int splits,
                                    rmsnorm_dtype_t dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_GEMV_MI355X_H */
