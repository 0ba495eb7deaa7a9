"""GPU outputs against relations the method fixes exactly, checked on the
library's own results (no oracle), up to the full bf16 4096 x 4096 workload in
the launch configuration the benchmark times.

Scaling by a power of two is exact in binary floating point, so wherever the
algebra of RMSNorm makes an output scale-equivariant, the kernels must
reproduce it bit for bit.  The algebra is that of "训推加速 Qwen3 实战：从
“调包”到手写 Triton Kernel（含 backward）": §4.1 (the forward,
y = w x / sqrt(mean(x^2) + eps)) and §5.3 (the backward, dx and dw):

  * eps = 0, x -> 4^k x:  y unchanged, rstd -> rstd / 4^k, dx -> dx / 4^k,
    dw unchanged (sum of squares scales by 16^k, its square root by 4^k);
  * any eps, x -> -x:     y -> -y, rstd and dx unchanged, dw -> -dw;
  * dy -> 2^m dy:         dx -> 2^m dx, dw -> 2^m dw (both linear in dy);
  * a row's outputs do not depend on the other rows of the batch;
  * dy = 0 with a residual-stream gradient: dh = dres and dw = 0 exactly;
  * rows = 1: dw_j = dy_j x_j rstd (one product per column, one rounding).
A dropped term, a wrong sign, a mixed-up row or column index breaks one of
these.  Inputs stay far from overflow and subnormals, where the relations
would stop being exact.
"""
import numpy as np
import pytest
import torch

from bwd_rmsnorm_fwd_amd import binding as B
from bwd_rmsnorm_fwd_amd import synth
from _gpu_util import DEV, f64, to_dev, torch_dtype, ulp_bf16

pytestmark = pytest.mark.gpu

DTYPES = [synth.BF16, synth.F32]
SHAPES = [(64, 896), (33, 4096), (300, 128), (9, 8192), (5, 897), (17, 129)]


def _scaled(a: np.ndarray, dtype: str, s: float) -> np.ndarray:
    """Host tensor of ``dtype`` multiplied by a power of two (exact)."""
    return synth.quantise(synth.to_f64(a, dtype).astype(np.float32) * np.float32(s), dtype)


def _run(x, w, dy, eps, dtype, rows, H):
    """fwd then bwd with the saved statistic; returns device tensors."""
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    td = torch_dtype(dtype)
    y = torch.full((rows, H), float("nan"), dtype=td, device=DEV)
    rstd = torch.full((rows,), float("nan"), device=DEV)
    dx = torch.full((rows, H), float("nan"), dtype=td, device=DEV)
    dw = torch.full((H,), float("nan"), dtype=td, device=DEV)
    code = B.F32 if dtype == synth.F32 else B.BF16
    ws = torch.empty(max(B.rmsnorm_bwd_workspace_bytes(rows, H, code), 16), dtype=torch.uint8,
                     device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, eps)
    B.rmsnorm_bwd(dyd, xd, wd, rstd, None, dx, dw, ws, eps)
    torch.cuda.synchronize()
    return y, rstd, dx, dw


def _host(*ts):
    return [f64(t) for t in ts]


def _same(name, a, b):
    assert not np.isnan(a).any(), f"{name}: NaN (output not written)"
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, f"{name}: {bad.size} elements differ, first at {bad[0]}"


@pytest.mark.parametrize("k", [-1, 1, 2])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", SHAPES)
def test_power_of_four_scaling_at_eps0(rows, H, dtype, k):
    wl = synth.small_case(rows, H, dtype, seed=rows + 13 * H, outlier_frac=0.01)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    s = 4.0 ** k
    a = _host(*_run(x, w, dy, 0.0, dtype, rows, H))
    b = _host(*_run(_scaled(x, dtype, s), w, dy, 0.0, dtype, rows, H))
    _same("y", b[0], a[0])
    _same("rstd", b[1] * s, a[1])
    _same("dx", b[2] * s, a[2])
    _same("dw", b[3], a[3])


def test_power_of_four_scaling_full_workload():
    """The bf16 4096 x 4096 workload (outlier feature columns included), as
    the benchmark launches it, at eps = 0."""
    wl = synth.WORKLOADS["c2_bf16_4096x4096"]
    x, w, dy = wl.x(), wl.w(), wl.dy()
    a = _host(*_run(x, w, dy, 0.0, wl.dtype, wl.rows, wl.H))
    b = _host(*_run(_scaled(x, wl.dtype, 4.0), w, dy, 0.0, wl.dtype, wl.rows, wl.H))
    _same("y", b[0], a[0])
    _same("rstd", b[1] * 4.0, a[1])
    _same("dx", b[2] * 4.0, a[2])
    _same("dw", b[3], a[3])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", SHAPES)
def test_sign_symmetry(rows, H, dtype):
    wl = synth.small_case(rows, H, dtype, seed=3 * rows + H)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    a = _host(*_run(x, w, dy, wl.eps, dtype, rows, H))
    b = _host(*_run(_scaled(x, dtype, -1.0), w, dy, wl.eps, dtype, rows, H))
    _same("y", -b[0], a[0])
    _same("rstd", b[1], a[1])
    _same("dx", b[2], a[2])
    _same("dw", -b[3], a[3])


@pytest.mark.parametrize("m", [-3, 1])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", SHAPES[:4])
def test_linear_in_dy(rows, H, dtype, m):
    wl = synth.small_case(rows, H, dtype, seed=5 * rows + 7 * H)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    s = 2.0 ** m
    a = _host(*_run(x, w, dy, wl.eps, dtype, rows, H))
    b = _host(*_run(x, w, _scaled(dy, dtype, s), wl.eps, dtype, rows, H))
    _same("y", b[0], a[0])
    _same("dx", b[2], a[2] * s)
    _same("dw", b[3], a[3] * s)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", [(300, 128), (64, 896), (40, 4096), (12, 8192), (33, 895)])
def test_rows_do_not_depend_on_the_batch(rows, H, dtype):
    """A sub-batch (a 16-byte aligned slice of rows) and a batch with one row
    changed give bitwise the same outputs on every other row."""
    wl = synth.small_case(rows, H, dtype, seed=rows * H % 9973)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    y, rstd, dx, _ = _host(*_run(x, w, dy, wl.eps, dtype, rows, H))
    lo, hi = 8, rows - 3
    ys, rs, dxs, _ = _host(*_run(x[lo:hi], w, dy[lo:hi], wl.eps, dtype, hi - lo, H))
    _same("y[sub]", ys, y[lo:hi])
    _same("rstd[sub]", rs, rstd[lo:hi])
    _same("dx[sub]", dxs, dx[lo:hi])
    k = rows // 2
    x2, dy2 = x.copy(), dy.copy()
    x2[k] = synth.normal(99, (H,), 3.0, dtype)
    dy2[k] = synth.normal(98, (H,), 1.0, dtype)
    y2, r2, dx2, _ = _host(*_run(x2, w, dy2, wl.eps, dtype, rows, H))
    keep = np.arange(rows) != k
    _same("y[other rows]", y2[keep], y[keep])
    _same("rstd[other rows]", r2[keep], rstd[keep])
    _same("dx[other rows]", dx2[keep], dx[keep])
    assert not np.array_equal(y2[k], y[k])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", [(64, 896), (16, 4096), (7, 8192), (300, 128), (5, 897)])
def test_residual_bwd_zero_dy_passes_dres_through(rows, H, dtype):
    wl = synth.small_case(rows, H, dtype, seed=rows + H, residual=True)
    x, res, w, dres = wl.x(), wl.res(), wl.w(), wl.dres()
    xd, rd, wd, drd = (to_dev(a, dtype) for a in (x, res, w, dres))
    td = torch_dtype(dtype)
    h = torch.empty((rows, H), dtype=td, device=DEV)
    y = torch.empty((rows, H), dtype=td, device=DEV)
    rstd = torch.empty(rows, device=DEV)
    B.rmsnorm_residual_fwd(xd, rd, wd, h, y, rstd, wl.eps)
    dy = torch.zeros((rows, H), dtype=td, device=DEV)
    dh = torch.full((rows, H), float("nan"), dtype=td, device=DEV)
    dw = torch.full((H,), float("nan"), dtype=td, device=DEV)
    code = B.F32 if dtype == synth.F32 else B.BF16
    ws = torch.empty(B.rmsnorm_bwd_workspace_bytes(rows, H, code), dtype=torch.uint8, device=DEV)
    B.rmsnorm_bwd(dy, h, wd, rstd, drd, dh, dw, ws, wl.eps)
    torch.cuda.synchronize()
    _same("dh", f64(dh), synth.to_f64(dres, dtype))
    _same("dw", f64(dw), np.zeros(H))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H", [1, 128, 896, 4096, 8192, 4095])
def test_single_row_dw_is_the_elementwise_product(H, dtype):
    wl = synth.small_case(1, H, dtype, seed=H + 17)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    _, rstd, _, dw = _host(*_run(x, w, dy, wl.eps, dtype, 1, H))
    exact = synth.to_f64(dy, dtype)[0] * synth.to_f64(x, dtype)[0] * rstd[0]
    err = np.abs(dw - exact)
    if dtype == synth.BF16:
        assert np.all(err <= ulp_bf16(exact)), float(np.max(err / ulp_bf16(exact)))
    else:
        assert np.all(err <= 2.0 ** -22 * np.abs(exact)), float(np.max(err / np.abs(exact)))
