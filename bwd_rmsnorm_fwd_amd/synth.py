"""Seeded synthetic inputs for the RMSNorm workloads.

This module only draws random numbers and quantises them to the I/O dtype; it
holds none of the normalisation arithmetic.  The same host arrays feed both
the HIP library (after a copy to the device) and the double-precision oracle
(after exact widening to float64).

Value recipes (the pages' workloads are real activations of the models they
train or decode; these synthetic stand-ins keep their shapes):
  * x ~ N(0, 1); w ~ U(0.5, 1.5); upstream gradients dy, dres ~ N(0, sigma).
  * "outlier features": ceil(1% of H) feature columns, chosen by a seeded
    permutation, are multiplied by 50 in every row before quantisation.
  * Quantisation to bfloat16 is round-to-nearest-even from float32.
Each tensor has its own seed (numpy PCG64), so any tensor can be regenerated
alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a host tensor stored in ``dtype``."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def quantise(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> host storage of ``dtype`` (uint16 bits for bf16)."""
    if dtype == BF16:
        return f32_to_bf16_bits(a32)
    return np.ascontiguousarray(a32, dtype=np.float32)


def normal(seed: int, shape, sigma: float = 1.0, dtype: str = BF16,
           outlier_cols: int = 0, outlier_seed: int = 0, outlier_scale: float = 50.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    if outlier_cols:
        H = shape[-1]
        cols = np.random.default_rng(outlier_seed).permutation(H)[:outlier_cols]
        a[..., cols] *= np.float32(outlier_scale)
    return quantise(a, dtype)


def uniform(seed: int, shape, lo: float = 0.5, hi: float = 1.5, dtype: str = BF16):
    rng = np.random.default_rng(seed)
    a = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return quantise(a, dtype)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, dtype, eps and per-tensor seeds."""
    name: str
    dtype: str
    rows: int
    H: int
    eps: float = 1e-6
    seed_x: int = 0
    seed_w: int = 0
    seed_dy: int = 0
    seed_res: int = 0
    seed_dres: int = 0
    x_outlier_frac: float = 0.0
    seed_outlier: int = 0
    dy_sigma: float = 1e-2
    residual: bool = False
    decode_splits: tuple = field(default_factory=tuple)

    @property
    def elems(self) -> int:
        return self.rows * self.H

    def x(self):
        k = int(math.ceil(self.x_outlier_frac * self.H)) if self.x_outlier_frac else 0
        return normal(self.seed_x, (self.rows, self.H), 1.0, self.dtype, k, self.seed_outlier)

    def w(self):
        return uniform(self.seed_w, (self.H,), 0.5, 1.5, self.dtype)

    def dy(self):
        return normal(self.seed_dy, (self.rows, self.H), self.dy_sigma, self.dtype)

    def res(self):
        return normal(self.seed_res, (self.rows, self.H), 1.0, self.dtype)

    def dres(self):
        return normal(self.seed_dres, (self.rows, self.H), self.dy_sigma, self.dtype)


# The five workloads of the pages' hot path (shapes from P1's B=4,T=4096,H=4096
# training rows and P2's hidden width 896 decode), as synthetic stand-ins.
WORKLOADS = {
    # fp32 I/O, small: rows=64, H=896; dy ~ N(0, 1).
    "c1_f32_64x896": Workload("c1_f32_64x896", F32, 64, 896, 1e-6, 101, 102, 103, dy_sigma=1.0),
    # bf16 training rows B=1,T=4096,H=4096 with 1% outlier feature columns x50.
    "c2_bf16_4096x4096": Workload("c2_bf16_4096x4096", BF16, 4096, 4096, 1e-6, 201, 202, 203,
                                  x_outlier_frac=0.01, seed_outlier=205),
    # bf16 decode, one row of width 896, split-row sum of squares.
    "c3_bf16_decode_1x896": Workload("c3_bf16_decode_1x896", BF16, 1, 896, 1e-6, 301, 302,
                                     decode_splits=(4, 8, 16)),
    # bf16 residual-add + RMSNorm, B=4,T=4096,H=4096.
    "c4_bf16_residual_16384x4096": Workload("c4_bf16_residual_16384x4096", BF16, 16384, 4096, 1e-6,
                                            401, 403, 404, 402, 405, residual=True),
    # bf16 narrow rows (several rows per wavefront).
    "c5a_bf16_262144x128": Workload("c5a_bf16_262144x128", BF16, 262144, 128, 1e-6, 501, 502, 503),
    # bf16 wide rows.
    "c5b_bf16_8192x8192": Workload("c5b_bf16_8192x8192", BF16, 8192, 8192, 1e-6, 511, 512, 513),
}


def small_case(rows: int, H: int, dtype: str = BF16, seed: int = 7, eps: float = 1e-6,
               dy_sigma: float = 1e-2, residual: bool = False, outlier_frac: float = 0.0) -> Workload:
    """A seeded workload of arbitrary shape for parity and edge-case tests."""
    s = 1000 * seed
    return Workload(f"case_{dtype}_{rows}x{H}_s{seed}", dtype, rows, H, eps,
                    s + 1, s + 2, s + 3, s + 4, s + 5, outlier_frac, s + 6, dy_sigma, residual)


@dataclass(frozen=True)
class GemvWorkload:
    """Decode projection y = A x: A [N][K] ~ N(0, sigma_a^2), x [K] ~ N(0, 1)."""
    name: str
    dtype: str
    N: int
    K: int
    seed_a: int
    seed_x: int
    sigma_a: float = 0.02
    splits: tuple = (1, 4, 8, 16)

    def A(self):
        return normal(self.seed_a, (self.N, self.K), self.sigma_a, self.dtype)

    def x(self):
        return normal(self.seed_x, (self.K,), 1.0, self.dtype)


# P2's q_proj at batch 1: hidden 896 -> 1024 outputs, split 1/4/8/16.
GEMV_WORKLOADS = {
    "q_proj_bf16_1024x896": GemvWorkload("q_proj_bf16_1024x896", BF16, 1024, 896, 601, 602),
}
