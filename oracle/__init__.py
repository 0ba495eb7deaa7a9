"""Oracle for fused row-wise RMSNorm: plain double-precision C loops.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library (``bwd_rmsnorm_fwd_amd``) and neither imports the other.

The arithmetic lives in ``rmsnorm_oracle.c`` (one plain loop nest per
operation, each citing the passage it restates).  This module only compiles it
with gcc and marshals numpy float64 arrays through ctypes.

Sources:
  P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）"
       (iqiancheng.github.io): §4.1 forward definition, §5.3 backward.
  P2 = trdm.cn/news/483216, hand-written Triton decode kernels: §2.1 the
       residual_add -> rms_norm pair and the planned fused kernel; §3.1 the
       decode projection y = A x (computed there with split-K).

Pinned by tests/test_oracle_pins.py (closed forms, invariants, central finite
differences, a hand-derived worked example and library rounding routines).
Every function here has at least one pin; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rmsnorm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

H_F32 = 0
H_BF16 = 1
H_EXACT = 2

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
        "-fno-fast-math", "-o", out + ".tmp", src, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # RMSNORM_ORACLE_LIB names another build of this source to load instead;
    # the mutation test uses it to run the pins against deliberately broken
    # copies of the oracle.
    path = os.environ.get("RMSNORM_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_double
    lib.oracle_round_f32.argtypes = [ctypes.c_double]
    lib.oracle_round_f32.restype = ctypes.c_double
    lib.oracle_rmsnorm_fwd.argtypes = [dp, dp, i64, i64, ctypes.c_double, dp, dp]
    lib.oracle_rmsnorm_fwd.restype = None
    lib.oracle_rmsnorm_residual_fwd.argtypes = [
        dp, dp, dp, i64, i64, ctypes.c_double, ctypes.c_int, dp, dp, dp]
    lib.oracle_rmsnorm_residual_fwd.restype = None
    lib.oracle_rmsnorm_bwd.argtypes = [dp, dp, dp, dp, dp, i64, i64, ctypes.c_double, dp, dp]
    lib.oracle_rmsnorm_bwd.restype = None
    lib.oracle_gemv.argtypes = [dp, dp, i64, i64, dp]
    lib.oracle_gemv.restype = None
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as2d(a, rows, H):
    a = np.ascontiguousarray(a, dtype=np.float64)
    assert a.size == rows * H, (a.shape, rows, H)
    return a.reshape(rows, H)


def round_bf16(v: float) -> float:
    return _load().oracle_round_bf16(float(v))


def round_f32(v: float) -> float:
    return _load().oracle_round_f32(float(v))


def rmsnorm_fwd(x, w, eps):
    """y = w * x * r per row, r = 1/sqrt(mean(x^2) + eps).  Returns (y, rstd)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, H = x.shape
    w = np.ascontiguousarray(w, dtype=np.float64)
    assert w.shape == (H,)
    y = np.empty_like(x)
    r = np.empty(rows, dtype=np.float64)
    _load().oracle_rmsnorm_fwd(_ptr(x), _ptr(w), rows, H, float(eps), _ptr(y), _ptr(r))
    return y, r


def rmsnorm_residual_fwd(x, res, w, eps, h_kind=H_BF16):
    """h = store(x + res); y = RMSNorm(h).  Returns (h, y, rstd)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, H = x.shape
    res = _as2d(res, rows, H)
    w = np.ascontiguousarray(w, dtype=np.float64)
    assert w.shape == (H,)
    h = np.empty_like(x)
    y = np.empty_like(x)
    r = np.empty(rows, dtype=np.float64)
    _load().oracle_rmsnorm_residual_fwd(
        _ptr(x), _ptr(res), _ptr(w), rows, H, float(eps), int(h_kind), _ptr(h), _ptr(y), _ptr(r))
    return h, y, r


def rmsnorm_bwd(dy, x, w, eps, rstd=None, dres=None):
    """dx (+dres) and dw.  rstd: saved statistic per row, or None to recompute."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, H = x.shape
    dy = _as2d(dy, rows, H)
    w = np.ascontiguousarray(w, dtype=np.float64)
    assert w.shape == (H,)
    if rstd is not None:
        rstd = np.ascontiguousarray(rstd, dtype=np.float64)
        assert rstd.shape == (rows,)
    if dres is not None:
        dres = _as2d(dres, rows, H)
    dx = np.empty_like(x)
    dw = np.empty(H, dtype=np.float64)
    _load().oracle_rmsnorm_bwd(
        _ptr(dy), _ptr(x), _ptr(w), _ptr(rstd), _ptr(dres), rows, H, float(eps), _ptr(dx), _ptr(dw))
    return dx, dw


def gemv(A, x):
    """y[n] = sum_k A[n][k] x[k] (plain dot products, natural order)."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    N, K = A.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.shape == (K,)
    y = np.empty(N, dtype=np.float64)
    _load().oracle_gemv(_ptr(A), _ptr(x), N, K, _ptr(y))
    return y
