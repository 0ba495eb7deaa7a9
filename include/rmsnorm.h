/*
 * rmsnorm.h -- C ABI of the fused row-wise RMSNorm library for AMD MI355X
 * (gfx950).  Library: librmsnorm_mi355x.so.
 *
 * Operation (restated from the sources below):
 *   forward   y[i][j] = w[j] * x[i][j] * r_i,  r_i = 1 / sqrt(mean_j x[i][j]^2 + eps)
 *   backward  wdy = w * dy;  c_i = (1/H) sum_j wdy[i][j] * x[i][j];
 *             dx[i][j] = r_i * (wdy[i][j] - x[i][j] * r_i^2 * c_i)
 *             dw[j]    = sum_i dy[i][j] * x[i][j] * r_i
 *   residual  h = x + res (stored in the I/O dtype), then y = forward(h)
 *
 * Sources:
 *   P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）"
 *        (iqiancheng.github.io): §4.1 forward definition, §4.2-4.3 forward
 *        kernel and wrapper, §5.3 backward derivation, §5.4 backward kernel
 *        and the two-pass dw, §5.6 gotchas (contiguous inputs, fp32
 *        reductions, no atomics for dw, eps is a plain float).
 *   P2 = trdm.cn/news/483216 (hand-written Triton decode kernels): §2.1 the
 *        residual_add / rms_norm pair and the planned fused kernel, §3.2
 *        split-K RMSNorm with a merge kernel, §3.3 fp32 partial sums and a
 *        fixed-order merge instead of atomics, §4.1-4.4 capture rules (no
 *        allocation, no host sync, one stream, stable addresses), §5.1 the
 *        merge must mask indices beyond the split count.
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" are HIP device (or managed) memory owned by the
 *     caller.  The library never allocates, frees or retains memory, so every
 *     call may be recorded into a HIP graph.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no
 *     call synchronises the host.  Results are valid once the stream reaches
 *     that point.
 *   - Tensors are dense and row-major: element (i, j) of a [rows][H] tensor is
 *     at offset i * H + j.  All tensor arguments of one call share `dtype`
 *     (rstd, workspace and partials are always fp32).
 *   - Each pointer must be aligned to its element size; 16-byte alignment of
 *     every pointer together with H * element_size % 16 == 0 selects the
 *     128-bit load/store path (otherwise a scalar path of the same kernels).
 *   - Arithmetic: inputs are widened to fp32; the per-row sums (sum of
 *     squares, c) accumulate in fp64; each output is rounded once to its
 *     dtype (round to nearest even).  dw accumulates in fp32.  Squares are
 *     formed in fp64 (exact for any finite input).  For bf16 I/O the
 *     backward's products w*dy*x are formed in fp32, where they are exact
 *     while 2^-126 <= |w*dy*x| < 2^128; the outputs themselves must be
 *     representable in the I/O dtype.
 *   - Non-finite inputs follow IEEE arithmetic of the definition within
 *     their row: a NaN in a row of x makes that row's y, rstd and dx NaN; an
 *     infinity gives r = 0 (y = 0, NaN where x is infinite; dx NaN).  dw sums
 *     over rows, so it is then NaN in every column.  Other rows are
 *     unaffected.
 *   - Reductions run in a fixed order and no float atomics are used: for a
 *     given shape, dtype and library build, results are bitwise identical
 *     from run to run.
 *   - Errors are reported by the return value only (nothing is printed and
 *     nothing aborts).  A call that returns anything but RMSNORM_OK enqueued
 *     no work, except RMSNORM_ELAUNCH, which reports a failure HIP returned
 *     for a launch.
 *   - Input and output buffers must not overlap, except where an entry
 *     point says otherwise.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of every tensor argument of a call (rstd/workspace: fp32). */
typedef enum {
    RMSNORM_F32 = 0,  /* IEEE binary32 */
    RMSNORM_BF16 = 1  /* bfloat16: 1 sign, 8 exponent, 7 fraction bits */
} rmsnorm_dtype_t;

typedef enum {
    RMSNORM_OK = 0,
    RMSNORM_EINVAL = 1,       /* null required pointer, rows < 0, H < 1, bad dtype,
                                 eps negative or not finite, bad split count */
    RMSNORM_EALIGN = 2,       /* a pointer is not aligned to its element size */
    RMSNORM_EWORKSPACE = 3,   /* workspace/partials missing or smaller than required */
    RMSNORM_EUNSUPPORTED = 4, /* H > RMSNORM_MAX_H, or H / vector width too large
                                 for the scalar path (see RMSNORM_MAX_H_SCALAR) */
    RMSNORM_ELAUNCH = 5,      /* HIP reported an error for a kernel launch */
    RMSNORM_ESCRATCH = 6      /* rmsnorm_bwd_noalloc: the shape needs more than the
                                 library's static scratch (RMSNORM_NOALLOC_SCRATCH_BYTES) */
} rmsnorm_status_t;

/* Largest row width.  Rows that miss the 128-bit path (odd H, unaligned
 * pointers) are limited to RMSNORM_MAX_H_SCALAR elements. */
#define RMSNORM_MAX_H 65536
#define RMSNORM_MAX_H_SCALAR 16384
/* Largest split count of rmsnorm_fwd_splitrow. */
#define RMSNORM_MAX_SPLITS 64

/* Forward: y = w * x * r per row, and the saved statistic rstd[i] = r_i
 * (P1 §4.1 definition, §4.2 kernel; saving r for the backward is the
 * alternative P1 §5.4 weighs against recomputing it).
 *   x     [rows][H] dtype, device, read
 *   w     [H]       dtype, device, read
 *   y     [rows][H] dtype, device, written
 *   rstd  [rows]    fp32,  device, written; may be NULL (not stored)
 *   rows >= 0 (0: no work), 1 <= H <= RMSNORM_MAX_H, eps >= 0 and finite.
 * Masked tail elements never contribute; the mean divides by H itself. */
rmsnorm_status_t rmsnorm_fwd(const void *x, const void *w, void *y, float *rstd,
                             int64_t rows, int64_t H, float eps,
                             rmsnorm_dtype_t dtype, hipStream_t stream);

/* Residual-add + RMSNorm forward (P2 §2.1: residual_add followed by rms_norm,
 * and the fused kernel planned there):
 *   h = x + res, rounded once to dtype and written out (the residual stream);
 *   y = w * h * r, r = 1 / sqrt(mean(h^2) + eps), computed from the stored
 *   (rounded) h, so the pair equals the unfused two-step sequence.
 *   x, res [rows][H] dtype, device, read;  w [H] dtype, device, read
 *   h, y   [rows][H] dtype, device, written;  rstd [rows] fp32 or NULL
 *   h may alias x or res (in-place residual update); y may not alias them. */
rmsnorm_status_t rmsnorm_residual_fwd(const void *x, const void *res, const void *w,
                                      void *h, void *y, float *rstd,
                                      int64_t rows, int64_t H, float eps,
                                      rmsnorm_dtype_t dtype, hipStream_t stream);

/* Bytes of device workspace rmsnorm_bwd needs for this shape: the fp32 dw
 * partial sums, one row of H per workgroup of the row pass.  Depends only on
 * (rows, H, dtype).  Returns 0 for rows == 0 or an invalid shape. */
size_t rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t H, rmsnorm_dtype_t dtype);

/* Backward (P1 §5.3 derivation, §5.4 two-pass dw without atomics):
 *   dx = r * (w*dy - x * r^2 * c) [+ dres],  c = (1/H) sum_j w_j dy_j x_j
 *   dw = sum over rows of dy * x * r, rounded once to dtype.
 *   dy    [rows][H] dtype, device, read (upstream gradient of y)
 *   x     [rows][H] dtype, device, read (the forward's input; h for the
 *                   residual variant)
 *   w     [H]       dtype, device, read
 *   rstd  [rows]    fp32, device, read: the statistic the forward saved; NULL
 *                   recomputes r from x with `eps` (P1 §5.4's choice)
 *   dres  [rows][H] dtype, device, read, may be NULL: gradient arriving on the
 *                   residual stream, added into dx.  With the residual
 *                   forward, dx is then the gradient of both x and res.
 *   dx    [rows][H] dtype, device, written (may alias dres or dy)
 *   dw    [H]       dtype, device, written (written as zeros when rows == 0)
 *   workspace       device, >= rmsnorm_bwd_workspace_bytes(rows, H, dtype),
 *                   16-byte aligned; contents are scratch, overwritten.
 * Runs rmsnorm_bwd_rows then rmsnorm_bwd_dw_reduce on `stream`. */
rmsnorm_status_t rmsnorm_bwd(const void *dy, const void *x, const void *w,
                             const float *rstd, const void *dres,
                             void *dx, void *dw, void *workspace, size_t workspace_bytes,
                             int64_t rows, int64_t H, float eps,
                             rmsnorm_dtype_t dtype, hipStream_t stream);

/* First pass of rmsnorm_bwd on its own: writes dx and the per-workgroup fp32
 * dw partial sums into `workspace`.  Arguments as for rmsnorm_bwd.
 * rows must be >= 1. */
rmsnorm_status_t rmsnorm_bwd_rows(const void *dy, const void *x, const void *w,
                                  const float *rstd, const void *dres, void *dx,
                                  void *workspace, size_t workspace_bytes,
                                  int64_t rows, int64_t H, float eps,
                                  rmsnorm_dtype_t dtype, hipStream_t stream);

/* Second pass of rmsnorm_bwd on its own: dw[j] = sum of the partial sums that
 * rmsnorm_bwd_rows left in `workspace` for the same (rows, H, dtype), added
 * in a fixed order and rounded once to dtype.  rows may be 0 (dw = 0). */
rmsnorm_status_t rmsnorm_bwd_dw_reduce(const void *workspace, size_t workspace_bytes,
                                       void *dw, int64_t rows, int64_t H,
                                       rmsnorm_dtype_t dtype, hipStream_t stream);

/* Bytes of the static device scratch behind rmsnorm_bwd_noalloc (one copy per
 * GPU the library runs on, held until the process ends): 256 partial rows of
 * 16384 floats, which covers every shape with H <= 16384, and wider rows
 * when rows is small enough (the need is rmsnorm_bwd_workspace_bytes). */
#define RMSNORM_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Backward for callers that cannot allocate device memory: code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Computes exactly what rmsnorm_bwd computes, with the same
 * kernels and reduction order (dx and dw bitwise equal to rmsnorm_bwd's),
 * but takes no workspace: the dw partial sums go to a scratch array that the
 * library holds in device memory, RMSNORM_NOALLOC_SCRATCH_BYTES per GPU.
 *   Arguments as for rmsnorm_bwd, without workspace/workspace_bytes.
 *   Returns RMSNORM_ESCRATCH, enqueuing nothing, when
 *   rmsnorm_bwd_workspace_bytes(rows, H, dtype) > RMSNORM_NOALLOC_SCRATCH_BYTES,
 *   RMSNORM_EINVAL when `stream` belongs to a device other than the current
 *   one (the scratch used is the current device's), and RMSNORM_ELAUNCH if
 *   HIP cannot give the scratch's device address.
 * No allocation of any kind: the scratch's address on the current device is
 * looked up once (hipGetSymbolAddress) on that device's first call.  Every
 * call on a GPU shares that GPU's one scratch array (the row pass overwrites
 * every partial the reduce pass reads, so nothing needs clearing): calls on
 * one GPU must not overlap in time (different streams or host threads
 * without ordering between them race on the scratch). */
rmsnorm_status_t rmsnorm_bwd_noalloc(const void *dy, const void *x, const void *w,
                                     const float *rstd, const void *dres,
                                     void *dx, void *dw, int64_t rows, int64_t H, float eps,
                                     rmsnorm_dtype_t dtype, hipStream_t stream);

/* Floats of partial sums rmsnorm_fwd_splitrow needs: rows * splits. */
size_t rmsnorm_splitrow_partials_count(int64_t rows, int splits);

/* Split-row forward for decode-sized batches (P2 §3.2 split-K RMSNorm; §3.3
 * fp32 partials and a fixed-order merge; §5.1 masked merge):
 *   pass 1: `splits` workgroups per row each write the fp32 sum of squares of
 *           one contiguous chunk of ceil(H / splits) elements to
 *           partials[i * splits + s];
 *   pass 2: a partial-reduce kernel adds the row's `splits` partials in index
 *           order (entries beyond `splits` are never read), forms r, writes
 *           rstd and y = w * x * r (P2's separate scale step is fused here).
 *   x, w, y, rstd: as rmsnorm_fwd (rstd may be NULL)
 *   partials  fp32, device, >= rmsnorm_splitrow_partials_count(rows, splits)
 *             floats (partials_count gives the size), scratch.
 *   1 <= splits <= RMSNORM_MAX_SPLITS; 1 <= rows.  splits == 1 is allowed.
 * The chunk sums are fp32 (the row's total is formed in fp64 from them). */
rmsnorm_status_t rmsnorm_fwd_splitrow(const void *x, const void *w, void *y, float *rstd,
                                      float *partials, size_t partials_count,
                                      int64_t rows, int64_t H, float eps, int splits,
                                      rmsnorm_dtype_t dtype, hipStream_t stream);

/* Static description of a status code.  Never NULL. */
const char *rmsnorm_status_str(rmsnorm_status_t status);

/* Dry run, per calling host thread (an introspection aid for benchmarks,
 * profilers and tests; not part of any passage of the sources).  While
 * enabled, every entry point of this library (decode_gemv_splitk included)
 * validates its arguments exactly as usual and returns the same status, but
 * instead of launching a kernel it appends one line per kernel it would
 * launch to a per-thread report:
 *     <kernel name with its template arguments> grid=<x>x<y>x<z> block=<n>
 * No device memory is touched and nothing is enqueued.  Returns the previous
 * setting (0 or 1); enabling clears the report. */
int rmsnorm_set_dry_run(int enable);

/* The calling thread's dry-run report since dry run was last enabled (an
 * empty string if nothing was recorded).  Owned by the library; valid until
 * the next call of any entry point on this thread. */
const char *rmsnorm_dry_run_report(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
