// Host launch loops for the benchmark: N back-to-back calls of one C entry
// point, made from C, so that a per-call time measured around them is the
// library's own (argument checks, dispatch, kernel launches) without the
// Python interpreter's per-call cost.  The entry point is passed in as a
// function pointer taken from the loaded library; this file calls nothing
// else and holds none of the method's arithmetic.
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

extern "C" {

typedef int (*fwd_fn)(const void*, const void*, void*, float*, int64_t, int64_t, float, int,
                      hipStream_t);
typedef int (*splitrow_fn)(const void*, const void*, void*, float*, float*, size_t, int64_t,
                           int64_t, float, int, int, hipStream_t);
typedef int (*bwd_fn)(const void*, const void*, const void*, const float*, const void*, void*,
                      void*, void*, size_t, int64_t, int64_t, float, int, hipStream_t);
typedef int (*gemv_fn)(const void*, const void*, void*, float*, size_t, int64_t, int64_t, int,
                       int, hipStream_t);

// Each returns 0, or the first non-zero status an entry point returned.
int bench_fwd_loop(void* fn, int n, const void* x, const void* w, void* y, float* rstd,
                   int64_t rows, int64_t H, float eps, int dtype, hipStream_t s) {
    fwd_fn f = (fwd_fn)fn;
    for (int i = 0; i < n; ++i) {
        const int st = f(x, w, y, rstd, rows, H, eps, dtype, s);
        if (st) return st;
    }
    return 0;
}

int bench_bwd_loop(void* fn, int n, const void* dy, const void* x, const void* w,
                   const float* rstd, const void* dres, void* dx, void* dw, void* ws,
                   size_t ws_bytes, int64_t rows, int64_t H, float eps, int dtype, hipStream_t s) {
    bwd_fn f = (bwd_fn)fn;
    for (int i = 0; i < n; ++i) {
        const int st = f(dy, x, w, rstd, dres, dx, dw, ws, ws_bytes, rows, H, eps, dtype, s);
        if (st) return st;
    }
    return 0;
}

int bench_splitrow_loop(void* fn, int n, const void* x, const void* w, void* y, float* rstd,
                        float* partials, size_t count, int64_t rows, int64_t H, float eps,
                        int splits, int dtype, hipStream_t s) {
    splitrow_fn f = (splitrow_fn)fn;
    for (int i = 0; i < n; ++i) {
        const int st = f(x, w, y, rstd, partials, count, rows, H, eps, splits, dtype, s);
        if (st) return st;
    }
    return 0;
}

int bench_gemv_loop(void* fn, int n, const void* A, const void* x, void* y, float* partials,
                    size_t count, int64_t N, int64_t K, int splits, int dtype, hipStream_t s) {
    gemv_fn f = (gemv_fn)fn;
    for (int i = 0; i < n; ++i) {
        const int st = f(A, x, y, partials, count, N, K, splits, dtype, s);
        if (st) return st;
    }
    return 0;
}

}  // extern "C"
