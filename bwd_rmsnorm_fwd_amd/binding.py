"""Python binding of librmsnorm_mi355x.so (C ABI in include/rmsnorm.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Functions take torch tensors that already live on the GPU, pass
their data pointers, shapes and torch's current HIP stream to the C entry
point of the same name, and raise ``RMSNormError`` on any status but OK.
PyTorch is used for device memory and streams; nothing here computes.

The library must have been built (``__graft_entry__.build()`` or
``python -m bwd_rmsnorm_fwd_amd._build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIB_PATH

OK, EINVAL, EALIGN, EWORKSPACE, EUNSUPPORTED, ELAUNCH, ESCRATCH = range(7)
NOALLOC_SCRATCH_BYTES = 16 << 20
F32, BF16 = 0, 1
MAX_H = 65536
MAX_H_SCALAR = 16384
MAX_SPLITS = 64

_lib = None


class RMSNormError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -m bwd_rmsnorm_fwd_amd._build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "rmsnorm_fwd": ([vp, vp, vp, vp, i64, i64, f32, i32, vp], i32),
        "rmsnorm_residual_fwd": ([vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp], i32),
        "rmsnorm_bwd_workspace_bytes": ([i64, i64, i32], sz),
        "rmsnorm_bwd": ([vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f32, i32, vp], i32),
        "rmsnorm_bwd_rows": ([vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f32, i32, vp], i32),
        "rmsnorm_bwd_dw_reduce": ([vp, sz, vp, i64, i64, i32, vp], i32),
        "rmsnorm_splitrow_partials_count": ([i64, i32], sz),
        "rmsnorm_fwd_splitrow": ([vp, vp, vp, vp, vp, sz, i64, i64, f32, i32, i32, vp], i32),
        "rmsnorm_status_str": ([i32], ctypes.c_char_p),
        "decode_gemv_partials_count": ([i64, i32], sz),
        "decode_gemv_splitk": ([vp, vp, vp, vp, sz, i64, i64, i32, i32, vp], i32),
        "rmsnorm_bwd_noalloc": ([vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp], i32),
        "rmsnorm_set_dry_run": ([i32], i32),
        "rmsnorm_dry_run_report": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().rmsnorm_status_str(int(status)).decode()


def rmsnorm_set_dry_run(enable: bool) -> bool:
    return bool(lib().rmsnorm_set_dry_run(1 if enable else 0))


def rmsnorm_dry_run_report() -> str:
    return lib().rmsnorm_dry_run_report().decode()


def launches_of(fn, *args) -> list:
    """The kernels (name, grid, block lines) that calling fn(*args) launches,
    recorded in the library's dry-run mode instead of launching them."""
    prev = rmsnorm_set_dry_run(True)
    try:
        fn(*args)
        return [l for l in rmsnorm_dry_run_report().splitlines() if l]
    finally:
        rmsnorm_set_dry_run(prev)


# ---------------------------------------------------------------- marshalling helpers

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _rows_h(x):
    if x.dim() < 1:
        raise ValueError("tensor must have at least one dimension")
    H = x.shape[-1]
    return (x.numel() // H if H else 0), H


def _expect(name, t, numel, dtype=None):
    """Refuse a tensor whose size or dtype does not match what the kernel
    will touch (the C ABI sees only pointers)."""
    if t is None:
        return
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")


def _check(fn, st):
    if st != OK:
        raise RMSNormError(fn, st)


def _contig(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (row-major [rows][H])")


# ---------------------------------------------------------------- entry points

def rmsnorm_fwd(x, w, y, rstd=None, eps: float = 1e-6, stream=None) -> None:
    """y = w * x / sqrt(mean(x^2) + eps) per row; rstd (fp32 [rows]) optional."""
    import torch
    _contig(x, w, y, rstd)
    rows, H = _rows_h(x)
    _expect("w", w, H, x.dtype)
    _expect("y", y, rows * H, x.dtype)
    _expect("rstd", rstd, rows, torch.float32)
    _check("rmsnorm_fwd", lib().rmsnorm_fwd(_p(x), _p(w), _p(y), _p(rstd), rows, H, float(eps),
                                            _dtype_code(x), _stream(stream)))


def rmsnorm_residual_fwd(x, res, w, h, y, rstd=None, eps: float = 1e-6, stream=None) -> None:
    """h = x + res (stored), y = RMSNorm(h)."""
    import torch
    _contig(x, res, w, h, y, rstd)
    rows, H = _rows_h(x)
    for name, t in (("res", res), ("h", h), ("y", y)):
        _expect(name, t, rows * H, x.dtype)
    _expect("w", w, H, x.dtype)
    _expect("rstd", rstd, rows, torch.float32)
    _check("rmsnorm_residual_fwd",
           lib().rmsnorm_residual_fwd(_p(x), _p(res), _p(w), _p(h), _p(y), _p(rstd), rows, H,
                                      float(eps), _dtype_code(x), _stream(stream)))


def rmsnorm_bwd_workspace_bytes(rows: int, H: int, dtype_code: int) -> int:
    return int(lib().rmsnorm_bwd_workspace_bytes(int(rows), int(H), int(dtype_code)))


def _bwd_expect(dy, x, w, rstd, dres, dx, rows, H):
    import torch
    for name, t in (("dy", dy), ("dres", dres), ("dx", dx)):
        _expect(name, t, rows * H, x.dtype)
    if dy is None or dx is None:
        raise ValueError("dy and dx are required")
    _expect("w", w, H, x.dtype)
    _expect("rstd", rstd, rows, torch.float32)


def rmsnorm_bwd(dy, x, w, rstd, dres, dx, dw, workspace, eps: float = 1e-6, stream=None) -> None:
    """dx (+dres) and dw; rstd None recomputes r; workspace: uint8 device tensor."""
    _contig(dy, x, w, rstd, dres, dx, dw, workspace)
    rows, H = _rows_h(x)
    _bwd_expect(dy, x, w, rstd, dres, dx, rows, H)
    _expect("dw", dw, H, x.dtype)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd",
           lib().rmsnorm_bwd(_p(dy), _p(x), _p(w), _p(rstd), _p(dres), _p(dx), _p(dw),
                             _p(workspace), nbytes, rows, H, float(eps), _dtype_code(x),
                             _stream(stream)))


def rmsnorm_bwd_noalloc(dy, x, w, rstd, dres, dx, dw, eps: float = 1e-6, stream=None) -> None:
    """As rmsnorm_bwd, with the dw partial sums in the library's static device
    scratch instead of a caller workspace (no allocation anywhere)."""
    _contig(dy, x, w, rstd, dres, dx, dw)
    rows, H = _rows_h(x)
    _bwd_expect(dy, x, w, rstd, dres, dx, rows, H)
    _expect("dw", dw, H, x.dtype)
    _check("rmsnorm_bwd_noalloc",
           lib().rmsnorm_bwd_noalloc(_p(dy), _p(x), _p(w), _p(rstd), _p(dres), _p(dx), _p(dw),
                                     rows, H, float(eps), _dtype_code(x), _stream(stream)))


def rmsnorm_bwd_rows(dy, x, w, rstd, dres, dx, workspace, eps: float = 1e-6, stream=None) -> None:
    _contig(dy, x, w, rstd, dres, dx, workspace)
    rows, H = _rows_h(x)
    _bwd_expect(dy, x, w, rstd, dres, dx, rows, H)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd_rows",
           lib().rmsnorm_bwd_rows(_p(dy), _p(x), _p(w), _p(rstd), _p(dres), _p(dx), _p(workspace),
                                  nbytes, rows, H, float(eps), _dtype_code(x), _stream(stream)))


def rmsnorm_bwd_dw_reduce(workspace, dw, rows: int, stream=None) -> None:
    _contig(workspace, dw)
    H = dw.numel()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd_dw_reduce",
           lib().rmsnorm_bwd_dw_reduce(_p(workspace), nbytes, _p(dw), int(rows), H,
                                       _dtype_code(dw), _stream(stream)))


def rmsnorm_splitrow_partials_count(rows: int, splits: int) -> int:
    return int(lib().rmsnorm_splitrow_partials_count(int(rows), int(splits)))


def rmsnorm_fwd_splitrow(x, w, y, rstd, partials, splits: int, eps: float = 1e-6,
                         stream=None) -> None:
    """Split-row forward: `splits` chunk sums per row, then the partial-reduce kernel."""
    import torch
    _contig(x, w, y, rstd, partials)
    rows, H = _rows_h(x)
    _expect("w", w, H, x.dtype)
    _expect("y", y, rows * H, x.dtype)
    _expect("rstd", rstd, rows, torch.float32)
    if partials is not None and partials.dtype != torch.float32:
        raise TypeError("partials must be float32")
    count = 0 if partials is None else partials.numel()
    _check("rmsnorm_fwd_splitrow",
           lib().rmsnorm_fwd_splitrow(_p(x), _p(w), _p(y), _p(rstd), _p(partials), count, rows, H,
                                      float(eps), int(splits), _dtype_code(x), _stream(stream)))


# ---------------------------------------------------------------- decode projection

def decode_gemv_partials_count(N: int, splits: int) -> int:
    return int(lib().decode_gemv_partials_count(int(N), int(splits)))


def decode_gemv_splitk(A, x, y, partials=None, splits: int = 1, stream=None) -> None:
    """y = A x (A [N][K]) with K split in `splits` segments (fp32 partials,
    then the fixed-order splitk_reduce pass)."""
    import torch
    _contig(A, x, y, partials)
    if A.dim() != 2:
        raise ValueError("A must be [N][K]")
    N, K = A.shape
    _expect("x", x, K, A.dtype)
    _expect("y", y, N, A.dtype)
    if partials is not None and partials.dtype != torch.float32:
        raise TypeError("partials must be float32")
    count = 0 if partials is None else partials.numel()
    _check("decode_gemv_splitk",
           lib().decode_gemv_splitk(_p(A), _p(x), _p(y), _p(partials), count, N, K, int(splits),
                                    _dtype_code(A), _stream(stream)))
