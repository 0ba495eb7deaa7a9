"""GPU parity of the split-K decode matrix-vector product against the oracle.

Bound (derived, none is stated for this path): products are exact and summed
in fp64 within a segment, each segment sum is rounded once to an fp32
partial, and the merged fp64 total is rounded once to the output dtype, so
|g - o| <= u(o) + 2^-24 * sum_s |p_s| <= u(o) + 2^-24 * sum_k |A_nk x_k|,
with u(o) one ulp of the output dtype at o (bf16: 8 significant bits; fp32:
24).  The tests use twice the second term."""
import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_fwd_amd import binding as B
from bwd_rmsnorm_fwd_amd import synth
from _gpu_util import DEV, f64, to_dev, torch_dtype, ulp_bf16

pytestmark = pytest.mark.gpu


def _bound(A64, x64, o, dtype):
    absdot = np.abs(A64) @ np.abs(x64)
    u = ulp_bf16(o) if dtype == synth.BF16 else np.abs(o) * 2.0 ** -23
    return u + 2.0 ** -23 * absdot


def _run(N, K, dtype, splits, seed):
    A = synth.normal(seed, (N, K), 0.02, dtype)
    x = synth.normal(seed + 1, (K,), 1.0, dtype)
    Ad, xd = to_dev(A, dtype), to_dev(x, dtype)
    y = torch.full((N,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    n = B.decode_gemv_partials_count(N, splits)
    parts = torch.full((n + 32,), float("nan"), device=DEV) if splits > 1 else None
    B.decode_gemv_splitk(Ad, xd, y, parts, splits)
    torch.cuda.synchronize()
    A64, x64 = synth.to_f64(A, dtype), synth.to_f64(x, dtype)
    o = oracle.gemv(A64, x64)
    g = f64(y)
    bad = np.abs(g - o) > _bound(A64, x64, o, dtype)
    assert not bad.any(), (np.flatnonzero(bad)[:5], g[bad][:5], o[bad][:5])
    if parts is not None:
        assert torch.isnan(parts[n:]).all()        # nothing past N * splits
    return y


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("N,K", [(1, 1), (7, 8), (64, 100), (300, 896), (1000, 4097), (33, 12288)])
@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8, 16, 64])
def test_gemv_parity(N, K, dtype, splits):
    _run(N, K, dtype, splits, seed=N * 31 + K)


@pytest.mark.parametrize("splits", [1, 4, 8, 16])
def test_q_proj_full_size(splits):
    wl = synth.GEMV_WORKLOADS["q_proj_bf16_1024x896"]
    y = _run(wl.N, wl.K, wl.dtype, splits, seed=wl.seed_a)
    y2 = _run(wl.N, wl.K, wl.dtype, splits, seed=wl.seed_a)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))   # deterministic
