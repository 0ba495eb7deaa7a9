"""Shared helpers for the GPU parity tests: host<->device transfer of seeded
inputs and the tolerance checks (not a test module)."""
from __future__ import annotations

import numpy as np
import torch

from bwd_rmsnorm_fwd_amd import synth

DEV = "cuda:0"


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Host storage from synth (uint16 bf16 bits or float32) -> device tensor."""
    if dtype == synth.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == synth.BF16 else torch.float32


def ulp_bf16(o: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at the magnitude of o (8 significant bits;
    fixed 2^-133 below 2^-126)."""
    a = np.abs(o)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126.0), -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def max_ulp_err_bf16(g: np.ndarray, o: np.ndarray) -> float:
    """max_i |g_i - o_i| / ulp_bf16(o_i)."""
    return float(np.max(np.abs(g - o) / ulp_bf16(o))) if g.size else 0.0


def normwise(g: np.ndarray, o: np.ndarray) -> float:
    """max_i |g_i - o_i| / max_i |o_i| (0 when o is all zero and g == o)."""
    if g.size == 0:
        return 0.0
    den = float(np.max(np.abs(o)))
    num = float(np.max(np.abs(g - o)))
    return num / den if den > 0 else num


# Tolerances (per tensor): fp32 I/O -> 2e-6 normwise on every output;
# bf16 I/O -> 1 bf16 ulp per element on y and dx (dh), bit-exact h,
# 1e-2 normwise on dw, and 2e-6 relative per element on the fp32 rstd.
F32_TOL = 2e-6
BF16_ULP = 1.0
BF16_DW_TOL = 1e-2
RSTD_REL = 2e-6


def assert_output(name: str, g: np.ndarray, o: np.ndarray, dtype: str):
    if dtype == synth.F32:
        err = normwise(g, o)
        assert err <= F32_TOL, f"{name}: normwise error {err:.3e} > {F32_TOL}"
    else:
        err = max_ulp_err_bf16(g, o)
        assert err <= BF16_ULP, f"{name}: {err:.3f} bf16 ulp > {BF16_ULP}"
    return err


def assert_dw(g: np.ndarray, o: np.ndarray, dtype: str):
    tol = F32_TOL if dtype == synth.F32 else BF16_DW_TOL
    err = normwise(g, o)
    assert err <= tol, f"dw: normwise error {err:.3e} > {tol}"
    return err


def assert_rstd(g: np.ndarray, o: np.ndarray):
    if g.size == 0:
        return 0.0
    err = float(np.max(np.abs(g - o) / np.abs(o)))
    assert err <= RSTD_REL, f"rstd: relative error {err:.3e} > {RSTD_REL}"
    return err


def round_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def oracle_stat(ro: np.ndarray):
    """The stored statistic taken from the oracle: the fp32 rounding of the
    oracle's double r (as float64 values for the oracle, and as a device fp32
    tensor for the library), so that both backwards get the same input and
    no expected value depends on a number the GPU produced."""
    r32 = round_f32(ro)
    return r32, torch.from_numpy(r32.astype(np.float32)).to(DEV)


def assert_rstd_rounded(g: np.ndarray, ro: np.ndarray):
    """The GPU forward's rstd must be the fp32 rounding of the oracle's r on
    every row (the row sums are exact products accumulated in fp64, so r is
    known to far more than fp32 precision on both sides)."""
    r32 = round_f32(ro)
    bad = np.flatnonzero(g != r32)
    assert bad.size == 0, (f"rstd differs from fp32(oracle r) on {bad.size} rows, first "
                           f"{bad[:5].tolist()}: {g[bad[:5]].tolist()} vs {r32[bad[:5]].tolist()}")
