"""Pins for the double-precision oracle (CPU only).

The oracle is checked against things other than itself: hand-derived worked
examples (tests/golden/worked_examples.txt), closed forms, invariants of the
mathematics, central finite differences of a scalar loss, and library rounding
routines.  Each pin is chosen so that a plausible slip in the oracle (dropped
eps, sum instead of mean, missing sqrt, wrong sign or power of r in dx, a
missing 1/H in c, a transposed weight index, dw without r, an unrounded
residual stream) fails at least one of them.

Sources: P1 = "训推加速 Qwen3 实战：从“调包”到手写 Triton Kernel（含 backward）"
(§4.1 forward, §5.3 backward, §5.6 gradcheck at (2, 32) in double);
P2 = trdm.cn/news/483216 (§2.1 residual_add -> rms_norm).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")


def _parse_golden(path):
    cases, cur = {}, None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
        elif key == "end":
            cases[cur["name"]] = cur
            cur = None
        else:
            cur[key] = [float(v) for v in vals]
    return cases


GOLD = _parse_golden(GOLDEN)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("name", ["h2_eps0", "h4_eps3", "two_rows_eps0"])
def test_golden_fwd_bwd(name):
    g = GOLD[name]
    rows, H = int(g["rows"][0]), int(g["H"][0])
    eps = g["eps"][0]
    x = np.array(g["x"]).reshape(rows, H)
    w = np.array(g["w"])
    dy = np.array(g["dy"]).reshape(rows, H)
    y, r = oracle.rmsnorm_fwd(x, w, eps)
    np.testing.assert_allclose(r, g["rstd"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(y.ravel(), g["y"], rtol=1e-15, atol=1e-300)
    dx, dw = oracle.rmsnorm_bwd(dy, x, w, eps)
    np.testing.assert_allclose(dx.ravel(), g["dx"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(dw, g["dw"], rtol=1e-15, atol=1e-15)
    # Same result when the forward's statistic is handed to the backward.
    dx2, dw2 = oracle.rmsnorm_bwd(dy, x, w, eps, rstd=r)
    np.testing.assert_allclose(dx2.ravel(), g["dx"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(dw2, g["dw"], rtol=1e-15, atol=1e-15)


def test_golden_residual_bf16_ties():
    g = GOLD["residual_bf16_ties"]
    H = int(g["H"][0])
    x = np.array(g["x"]).reshape(1, H)
    res = np.array(g["res"]).reshape(1, H)
    w = np.array(g["w"])
    h, y, r = oracle.rmsnorm_residual_fwd(x, res, w, g["eps"][0], oracle.H_BF16)
    assert h.ravel().tolist() == g["h"]            # bit-exact rounding, ties to even
    np.testing.assert_allclose(r, g["rstd"], rtol=1e-15)
    np.testing.assert_allclose(y.ravel(), g["y"], rtol=1e-15)
    # Without rounding the stream differs (a plain sum would give 1.00390625).
    h_exact, _, _ = oracle.rmsnorm_residual_fwd(x, res, w, 0.0, oracle.H_EXACT)
    assert h_exact[0, 0] == 1.00390625 and h_exact[0, 1] == 1.01171875


# ---------------------------------------------------------------- forward closed forms

@pytest.mark.parametrize("H", [1, 7, 896])
@pytest.mark.parametrize("c", [-3.0, -0.1, 1e-3, 0.1, 2.5])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_constant_row(H, c, eps):
    """x = c everywhere: mean of squares is c^2, so y = w c / sqrt(c^2 + eps)."""
    w = _rng(1).uniform(0.5, 1.5, H)
    y, r = oracle.rmsnorm_fwd(np.full((1, H), c), w, eps)
    expect = w * c / math.sqrt(c * c + eps)
    # A sequential double sum of H equal terms is good to about H * 2^-53.
    np.testing.assert_allclose(y[0], expect, rtol=1e-13)
    np.testing.assert_allclose(r[0], 1.0 / math.sqrt(c * c + eps), rtol=1e-13)
    if eps == 0.0:
        np.testing.assert_allclose(y[0], math.copysign(1.0, c) * w, rtol=1e-13)


def test_h1_closed_form():
    rng = _rng(2)
    for eps in (1e-6, 0.5):
        x = rng.standard_normal((5, 1))
        w = rng.uniform(0.5, 1.5, 1)
        dy = rng.standard_normal((5, 1))
        y, _ = oracle.rmsnorm_fwd(x, w, eps)
        np.testing.assert_allclose(y, w * x / np.sqrt(x * x + eps), rtol=1e-14)
        dx, dw = oracle.rmsnorm_bwd(dy, x, w, eps)
        # d/dx [w x / sqrt(x^2+eps)] = w eps / (x^2+eps)^(3/2).  The two terms
        # of the backward formula cancel to a relative eps/(x^2+eps), so the
        # bound is on the scale of the terms, |r w dy|.
        term = np.abs(w * dy / np.sqrt(x * x + eps))
        assert np.all(np.abs(dx - w * dy * eps / (x * x + eps) ** 1.5) <= 1e-14 * term)
        np.testing.assert_allclose(dw, [np.sum(dy * x / np.sqrt(x * x + eps))], rtol=1e-13)


def test_scale_invariance_eps0():
    """At eps = 0, y(a x) = sign(a) y(x); bit-identical for a = +-4^k."""
    rng = _rng(3)
    x = rng.standard_normal((6, 37))
    w = rng.uniform(0.5, 1.5, 37)
    y, _ = oracle.rmsnorm_fwd(x, w, 0.0)
    for a in (4.0, 0.25, -16.0, 1024.0):
        ya, _ = oracle.rmsnorm_fwd(a * x, w, 0.0)
        assert np.array_equal(ya, math.copysign(1.0, a) * y)
    for a in (3.7, -0.013):
        ya, _ = oracle.rmsnorm_fwd(a * x, w, 0.0)
        np.testing.assert_allclose(ya, math.copysign(1.0, a) * y, rtol=1e-14)


def test_unit_rms_invariant():
    """At eps = 0 each row of y/w has mean square exactly 1."""
    rng = _rng(4)
    x = rng.standard_normal((9, 129)) * 3.0
    w = rng.uniform(0.5, 1.5, 129)
    y, _ = oracle.rmsnorm_fwd(x, w, 0.0)
    np.testing.assert_allclose(np.mean((y / w) ** 2, axis=1), 1.0, rtol=1e-14)


def test_rows_independent_and_columns_equivariant():
    rng = _rng(5)
    x = rng.standard_normal((7, 33))
    w = rng.uniform(0.5, 1.5, 33)
    dy = rng.standard_normal((7, 33))
    y, r = oracle.rmsnorm_fwd(x, w, 1e-6)
    dx, _ = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
    x2 = x.copy()
    x2[3] = rng.standard_normal(33) * 10
    y2, _ = oracle.rmsnorm_fwd(x2, w, 1e-6)
    dx2, _ = oracle.rmsnorm_bwd(dy, x2, w, 1e-6)
    keep = [i for i in range(7) if i != 3]
    assert np.array_equal(y[keep], y2[keep]) and np.array_equal(dx[keep], dx2[keep])
    assert not np.allclose(y[3], y2[3])
    perm = rng.permutation(33)
    yp, rp = oracle.rmsnorm_fwd(x[:, perm], w[perm], 1e-6)
    np.testing.assert_allclose(yp, y[:, perm], rtol=1e-14)
    np.testing.assert_allclose(rp, r, rtol=1e-14)
    dxp, dwp = oracle.rmsnorm_bwd(dy[:, perm], x[:, perm], w[perm], 1e-6)
    _, dw = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
    np.testing.assert_allclose(dxp, dx[:, perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dwp, dw[perm], rtol=1e-12)


# ---------------------------------------------------------------- backward invariants

@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.3])
def test_x_dot_dx_identity(eps):
    """sum_j x_j dx_j = H c eps r^3 (derived from P1 §5.3); zero at eps = 0."""
    rng = _rng(6)
    rows, H = 5, 64
    x = rng.standard_normal((rows, H))
    w = rng.uniform(0.5, 1.5, H)
    dy = rng.standard_normal((rows, H))
    dx, _ = oracle.rmsnorm_bwd(dy, x, w, eps)
    lhs = np.sum(x * dx, axis=1)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    c = np.mean(w * dy * x, axis=1)
    scale = np.sum(np.abs(x * dx), axis=1)
    np.testing.assert_allclose(lhs, H * c * eps * r ** 3, rtol=0, atol=1e-13 * scale.max())
    if eps == 0.0:
        assert np.all(np.abs(lhs) <= 1e-13 * scale)


def test_dw_ties_forward_and_backward():
    """dw_j w_j = sum over rows of dy_j y_j."""
    rng = _rng(7)
    x = rng.standard_normal((11, 40))
    w = rng.uniform(0.5, 1.5, 40)
    dy = rng.standard_normal((11, 40))
    y, _ = oracle.rmsnorm_fwd(x, w, 1e-6)
    _, dw = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
    np.testing.assert_allclose(dw * w, np.sum(dy * y, axis=0), rtol=1e-13)


def test_single_row_dw_and_constant_row_dx():
    rng = _rng(8)
    x = rng.standard_normal((1, 19))
    w = rng.uniform(0.5, 1.5, 19)
    dy = rng.standard_normal((1, 19))
    _, r = oracle.rmsnorm_fwd(x, w, 1e-6)
    _, dw = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
    np.testing.assert_allclose(dw, dy[0] * x[0] * r[0], rtol=1e-15)
    # Constant row c at eps = 0: dx = (wdy - mean(wdy)) / |c|.
    c = -1.75
    xc = np.full((1, 19), c)
    dxc, _ = oracle.rmsnorm_bwd(dy, xc, w, 0.0)
    wdy = w * dy[0]
    np.testing.assert_allclose(dxc[0], (wdy - wdy.mean()) / abs(c), rtol=1e-12, atol=1e-14)


def test_linear_in_dy_and_inverse_scale_in_x():
    rng = _rng(9)
    x = rng.standard_normal((4, 24))
    w = rng.uniform(0.5, 1.5, 24)
    d1 = rng.standard_normal((4, 24))
    d2 = rng.standard_normal((4, 24))
    a1, b1 = oracle.rmsnorm_bwd(d1, x, w, 1e-6)
    a2, b2 = oracle.rmsnorm_bwd(d2, x, w, 1e-6)
    a3, b3 = oracle.rmsnorm_bwd(2.0 * d1 - 3.0 * d2, x, w, 1e-6)
    np.testing.assert_allclose(a3, 2 * a1 - 3 * a2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b3, 2 * b1 - 3 * b2, rtol=1e-12, atol=1e-13)
    # eps = 0: dx(a x) = dx(x) / a.
    e1, _ = oracle.rmsnorm_bwd(d1, x, w, 0.0)
    e2, _ = oracle.rmsnorm_bwd(d1, 8.0 * x, w, 0.0)
    np.testing.assert_allclose(e2, e1 / 8.0, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- finite differences

def _loss(x, w, eps, g):
    y, _ = oracle.rmsnorm_fwd(x, w, eps)
    return float(np.sum(g * y))


@pytest.mark.parametrize("rows", [1, 2, 3])
@pytest.mark.parametrize("H", [1, 2, 3, 5, 8, 32])
@pytest.mark.parametrize("eps", [1e-6, 0.1])
def test_central_finite_differences(rows, H, eps):
    """dx and dw equal the central differences of L = sum(g * y) (a random
    scalar loss), in double -- the role of P1 §5.6's double gradcheck."""
    rng = _rng(100 + 10 * rows + H)
    x = rng.standard_normal((rows, H))
    w = rng.uniform(0.5, 1.5, H)
    g = rng.standard_normal((rows, H))
    dx, dw = oracle.rmsnorm_bwd(g, x, w, eps)
    h = 1e-6
    num_dx = np.zeros_like(x)
    for i in range(rows):
        for j in range(H):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            num_dx[i, j] = (_loss(xp, w, eps, g) - _loss(xm, w, eps, g)) / (2 * h)
    num_dw = np.zeros_like(w)
    for j in range(H):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        num_dw[j] = (_loss(x, wp, eps, g) - _loss(x, wm, eps, g)) / (2 * h)
    np.testing.assert_allclose(dx, num_dx, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw, num_dw, rtol=1e-6, atol=1e-8)


def test_gradcheck_shape_of_the_page():
    """P1 §5.6 runs a double-precision gradcheck at x (2, 32), eps 1e-6 with
    atol 1e-4; the same check against central differences."""
    rng = _rng(11)
    x = rng.standard_normal((2, 32))
    w = rng.standard_normal(32)
    g = rng.standard_normal((2, 32))
    dx, dw = oracle.rmsnorm_bwd(g, x, w, 1e-6)
    h = 1e-6
    for i in range(2):
        for j in range(32):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            num = (_loss(xp, w, 1e-6, g) - _loss(xm, w, 1e-6, g)) / (2 * h)
            assert abs(num - dx[i, j]) <= 1e-4 + 1e-3 * abs(num)
    for j in range(32):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        num = (_loss(x, wp, 1e-6, g) - _loss(x, wm, 1e-6, g)) / (2 * h)
        assert abs(num - dw[j]) <= 1e-4 + 1e-3 * abs(num)


def test_residual_backward_by_finite_differences():
    """Unrounded residual stream: d/dx = d/dres = the norm's dx at h, and the
    incoming residual-stream gradient adds straight through."""
    rng = _rng(12)
    rows, H, eps = 3, 6, 1e-3
    x = rng.standard_normal((rows, H))
    res = rng.standard_normal((rows, H))
    w = rng.uniform(0.5, 1.5, H)
    g = rng.standard_normal((rows, H))       # upstream grad of y
    gh = rng.standard_normal((rows, H))      # upstream grad of h (residual stream)

    def L(xx, rr):
        hh, yy, _ = oracle.rmsnorm_residual_fwd(xx, rr, w, eps, oracle.H_EXACT)
        return float(np.sum(g * yy) + np.sum(gh * hh))

    hcur, _, r = oracle.rmsnorm_residual_fwd(x, res, w, eps, oracle.H_EXACT)
    dh, _ = oracle.rmsnorm_bwd(g, hcur, w, eps, rstd=r, dres=gh)
    step = 1e-6
    for i in range(rows):
        for j in range(H):
            for which in (0, 1):
                a, b = x.copy(), res.copy()
                tgt = a if which == 0 else b
                tgt[i, j] += step
                lp = L(a, b)
                tgt[i, j] -= 2 * step
                lm = L(a, b)
                assert abs((lp - lm) / (2 * step) - dh[i, j]) < 1e-7 * (1 + abs(dh[i, j]))


def test_residual_dy_zero_gives_dres_exactly():
    rng = _rng(13)
    x = rng.standard_normal((4, 10))
    w = rng.uniform(0.5, 1.5, 10)
    dres = rng.standard_normal((4, 10))
    dh, dw = oracle.rmsnorm_bwd(np.zeros((4, 10)), x, w, 1e-6, dres=dres)
    assert np.array_equal(dh, dres) and np.all(dw == 0)


def test_saved_rstd_is_used():
    """A supplied statistic replaces the recomputed one (the bwd is then
    linear in it for the c term): dx(rstd = 2r) follows the formula."""
    rng = _rng(14)
    x = rng.standard_normal((3, 16))
    w = rng.uniform(0.5, 1.5, 16)
    dy = rng.standard_normal((3, 16))
    _, r = oracle.rmsnorm_fwd(x, w, 1e-6)
    dx1, dw1 = oracle.rmsnorm_bwd(dy, x, w, 1e-6, rstd=r)
    dx0, dw0 = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
    assert np.array_equal(dx1, dx0) and np.array_equal(dw1, dw0)
    dx2, dw2 = oracle.rmsnorm_bwd(dy, x, w, 1e-6, rstd=2 * r)
    np.testing.assert_allclose(dw2, 2 * dw1, rtol=1e-14)
    # dx is not a multiple of dx1: the r^3 term scales by 8, the r term by 2.
    assert not np.allclose(dx2, 2 * dx1)


# ---------------------------------------------------------------- rounding helpers

def test_round_bf16_matches_library():
    """The oracle's bf16 rounding equals torch's float32 -> bfloat16 cast
    (round to nearest, ties to even) on random, tie, subnormal and overflow
    values."""
    rng = _rng(15)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3 * 2 ** -134, 2 ** -149,
                    3.3895313892515355e38, 3.39e38, -3.4e38, 0.0, -0.0, 1.0, 65504.0]),
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(float(v)) for v in vals])
    same = (got == ref) | (np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref)))
    assert same.all(), vals[~same][:10]


def test_round_f32_matches_library():
    rng = _rng(16)
    vals = rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 40, 5000)
    ref = vals.astype(np.float32).astype(np.float64)
    got = np.array([oracle.round_f32(float(v)) for v in vals])
    assert np.array_equal(got, ref)


def test_residual_bf16_equals_library_add_then_cast():
    """h from bf16 x and res equals torch's float64 add cast to bfloat16."""
    rng = _rng(17)
    x = torch.from_numpy(rng.standard_normal((8, 64)).astype(np.float32)).to(torch.bfloat16)
    r = torch.from_numpy((rng.standard_normal((8, 64)) * 10.0 ** rng.integers(-6, 3, (8, 64))).astype(np.float32)).to(torch.bfloat16)
    ref = (x.double() + r.double()).float().to(torch.bfloat16).double().numpy()
    w = np.ones(64)
    h, y, rs = oracle.rmsnorm_residual_fwd(x.double().numpy(), r.double().numpy(), w, 1e-6, oracle.H_BF16)
    assert np.array_equal(h, ref)
    y2, rs2 = oracle.rmsnorm_fwd(h, w, 1e-6)
    assert np.array_equal(y, y2) and np.array_equal(rs, rs2)


# ---------------------------------------------------------------- decode projection

def test_gemv_identity_and_constant():
    """A = I gives y = x; a constant matrix gives y_n = c * sum(x)."""
    rng = _rng(20)
    x = rng.standard_normal(37)
    assert np.array_equal(oracle.gemv(np.eye(37), x), x)
    y = oracle.gemv(np.full((5, 37), 0.25), x)
    np.testing.assert_allclose(y, 0.25 * np.sum(x), rtol=1e-13)


def test_gemv_matches_library_matmul():
    rng = _rng(21)
    A = rng.standard_normal((64, 896))
    x = rng.standard_normal(896)
    np.testing.assert_allclose(oracle.gemv(A, x), A @ x, rtol=1e-12, atol=1e-12)


def test_gemv_worked_example_and_linearity():
    # [[1, 2, 3], [4, 5, 6]] @ [1, -1, 2] = [1 - 2 + 6, 4 - 5 + 12] = [5, 11]
    A = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    assert oracle.gemv(A, np.array([1.0, -1.0, 2.0])).tolist() == [5.0, 11.0]
    rng = _rng(22)
    A = rng.standard_normal((9, 13))
    u, v = rng.standard_normal(13), rng.standard_normal(13)
    np.testing.assert_allclose(oracle.gemv(A, 2 * u - 3 * v),
                               2 * oracle.gemv(A, u) - 3 * oracle.gemv(A, v), rtol=1e-12, atol=1e-12)
    # Row n of the output depends on row n of A only (no transposed index).
    A2 = A.copy()
    A2[4] *= -1
    y, y2 = oracle.gemv(A, u), oracle.gemv(A2, u)
    assert y2[4] == -y[4] and np.array_equal(np.delete(y, 4), np.delete(y2, 4))
