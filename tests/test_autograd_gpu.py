"""The torch.autograd binding over the C ABI: gradients against the oracle,
the residual pair's two gradients, a gradcheck in the shape of P1 §5.6, and
the refusal of second-order gradients."""
import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_fwd_amd import synth
from bwd_rmsnorm_fwd_amd.autograd import RMSNorm, residual_rms_norm, rms_norm
from _gpu_util import DEV, assert_dw, assert_output, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_autograd_matches_oracle(dtype):
    B_, T, H = 2, 37, 896
    wl = synth.small_case(B_ * T, H, dtype, seed=31)
    x = to_dev(wl.x(), dtype).view(B_, T, H).requires_grad_(True)
    w = to_dev(wl.w(), dtype).requires_grad_(True)
    g = to_dev(wl.dy(), dtype).view(B_, T, H)
    y = rms_norm(x, w, wl.eps)
    y.backward(g)
    torch.cuda.synchronize()
    x64, w64, g64 = (synth.to_f64(a, dtype) for a in (wl.x(), wl.w(), wl.dy()))
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    assert_output("y", f64(y).reshape(-1, H), yo, dtype)
    dxo, dwo = oracle.rmsnorm_bwd(g64, x64, w64, wl.eps, rstd=ro.astype(np.float32).astype(np.float64))
    assert_output("dx", f64(x.grad).reshape(-1, H), dxo, dtype)
    assert_dw(f64(w.grad), dwo, dtype)


def test_residual_autograd_both_streams():
    """loss = sum(g*y) + sum(gh*h): x.grad == res.grad == dres + dx_norm."""
    rows, H, dtype = 64, 4096, synth.BF16
    wl = synth.small_case(rows, H, dtype, seed=32)
    x = to_dev(wl.x(), dtype).requires_grad_(True)
    res = to_dev(wl.res(), dtype).requires_grad_(True)
    w = to_dev(wl.w(), dtype).requires_grad_(True)
    g, gh = to_dev(wl.dy(), dtype), to_dev(wl.dres(), dtype)
    y, h = residual_rms_norm(x, res, w, wl.eps)
    ((y.float() * g.float()).sum() + (h.float() * gh.float()).sum()).backward()
    torch.cuda.synchronize()
    assert torch.equal(x.grad.view(torch.int16), res.grad.view(torch.int16))
    ho, yo, ro = oracle.rmsnorm_residual_fwd(synth.to_f64(wl.x(), dtype), synth.to_f64(wl.res(), dtype),
                                             synth.to_f64(wl.w(), dtype), wl.eps, oracle.H_BF16)
    assert np.array_equal(f64(h), ho)
    dho, dwo = oracle.rmsnorm_bwd(synth.to_f64(wl.dy(), dtype), ho, synth.to_f64(wl.w(), dtype),
                                  wl.eps, rstd=ro.astype(np.float32).astype(np.float64),
                                  dres=synth.to_f64(wl.dres(), dtype))
    assert_output("dh", f64(x.grad), dho, dtype)
    assert_dw(f64(w.grad), dwo, dtype)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradcheck_page_shape_fp32(seed):
    """P1 §5.6 runs gradcheck at x (2, 32), eps 1e-6.  The library has no
    fp64 I/O, so this is the fp32 version: the analytic backward against
    central differences of the GPU forward.  Tolerances follow from the
    arithmetic: y is the fp32 rounding of an exact value, so a difference
    quotient over 2h = 8e-3 carries about 6e-8 |y| / 4e-3 = 1.5e-5 of
    rounding, and the h^2 truncation term is a few 1e-6 at these magnitudes
    (the same differences of an fp64 forward rounded to fp32, on the host,
    stay within 4e-5 + 1e-3 of the exact Jacobian for five seeds); a slip in
    the backward of 1e-3 relative or more fails."""
    torch.manual_seed(seed)
    x = torch.randn(2, 32, device=DEV, dtype=torch.float32, requires_grad=True)
    w = torch.randn(32, device=DEV, dtype=torch.float32, requires_grad=True)
    assert torch.autograd.gradcheck(lambda a, b: rms_norm(a, b, 1e-6), (x, w), eps=4e-3,
                                    atol=2e-4, rtol=1e-3, nondet_tol=0.0, fast_mode=False)


def test_module_and_no_double_backward():
    m = RMSNorm(128, dtype=torch.bfloat16)
    x = torch.randn(4, 128, device=DEV, dtype=torch.bfloat16, requires_grad=True)
    y = m(x)
    gx, = torch.autograd.grad(y.float().sum(), x, create_graph=True)
    with pytest.raises(RuntimeError):
        gx.float().sum().backward()
