"""GPU parity: the HIP library (through the C ABI) against the double-precision
oracle, element by element, on seeded inputs.

Shapes span several tiles and ragged tails on both the 128-bit path and the
scalar path (odd H, unaligned pointers), every team width of the dispatch
table, and the degenerate cases (rows = 0, H = 1).  Full-size workloads are in
test_parity_full_gpu.py.

Tolerances: fp32 I/O 2e-6 normwise per tensor; bf16 I/O 1 bf16 ulp per element
on y and dx, bit-exact h, 1e-2 normwise on dw; fp32 rstd 2e-6 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_fwd_amd import binding as B
from bwd_rmsnorm_fwd_amd import synth
from _gpu_util import (DEV, assert_dw, assert_output, assert_rstd, assert_rstd_rounded, f64,
                       oracle_stat, round_f32, to_dev, torch_dtype)

pytestmark = pytest.mark.gpu

# (rows, H): tails of every team width, several tiles, vector and scalar paths.
SHAPES = [(1, 1), (3, 2), (5, 7), (64, 8), (65, 16), (33, 120), (257, 128), (17, 129),
          (9, 256), (7, 500), (70, 512), (11, 895), (64, 896), (5, 897), (6, 1024),
          (4, 2040), (3, 2048), (6, 1500), (9, 3000), (5, 4095), (7, 4096), (3, 5000), (2, 8192),
          (2, 16384)]
DTYPES = [synth.BF16, synth.F32]


def _inputs(rows, H, dtype, seed, outliers=0.0):
    wl = synth.small_case(rows, H, dtype, seed=seed, outlier_frac=outliers)
    return wl, wl.x(), wl.w(), wl.dy(), wl.res(), wl.dres()


def _empty(rows, H, dtype):
    return torch.full((rows, H), float("nan"), dtype=torch_dtype(dtype), device=DEV)


def _ws(rows, H, dtype):
    code = B.F32 if dtype == synth.F32 else B.BF16
    n = B.rmsnorm_bwd_workspace_bytes(rows, H, code)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", SHAPES)
def test_fwd(rows, H, dtype):
    wl, x, w, *_ = _inputs(rows, H, dtype, seed=rows * 7 + H, outliers=0.01)
    xd, wd = to_dev(x, dtype), to_dev(w, dtype)
    y = _empty(rows, H, dtype)
    rstd = torch.full((rows,), float("nan"), device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
    torch.cuda.synchronize()
    yo, ro = oracle.rmsnorm_fwd(synth.to_f64(x, dtype), synth.to_f64(w, dtype), wl.eps)
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", SHAPES[::2])
def test_residual_fwd(rows, H, dtype):
    wl, x, w, _, res, _ = _inputs(rows, H, dtype, seed=rows + 3 * H)
    xd, rd, wd = to_dev(x, dtype), to_dev(res, dtype), to_dev(w, dtype)
    h, y = _empty(rows, H, dtype), _empty(rows, H, dtype)
    rstd = torch.full((rows,), float("nan"), device=DEV)
    B.rmsnorm_residual_fwd(xd, rd, wd, h, y, rstd, wl.eps)
    torch.cuda.synchronize()
    kind = oracle.H_BF16 if dtype == synth.BF16 else oracle.H_F32
    ho, yo, ro = oracle.rmsnorm_residual_fwd(synth.to_f64(x, dtype), synth.to_f64(res, dtype),
                                             synth.to_f64(w, dtype), wl.eps, kind)
    assert np.array_equal(f64(h), ho), "h must be bit-exact"
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("mode", ["saved_rstd", "recompute", "dres"])
@pytest.mark.parametrize("rows,H", SHAPES)
def test_bwd(rows, H, dtype, mode):
    """The backward with the saved statistic (fp32 rstd) as its input on both
    sides, with r recomputed from x, and with a residual-stream gradient."""
    wl, x, w, dy, _, dres = _inputs(rows, H, dtype, seed=5 * rows + H, outliers=0.01)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    _, r64 = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    rstd32 = round_f32(r64)                      # the stored statistic, from the oracle
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    rstd_d = torch.from_numpy(rstd32.astype(np.float32)).to(DEV) if mode != "recompute" else None
    dres_d = to_dev(dres, dtype) if mode == "dres" else None
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_bwd(dyd, xd, wd, rstd_d, dres_d, dx, dw, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps,
                                  rstd=None if mode == "recompute" else rstd32,
                                  dres=synth.to_f64(dres, dtype) if mode == "dres" else None)
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


# Row counts that give the backward's 256 workgroups several row blocks each,
# unequal between workgroups, with a partly filled last block: the loop that
# alternates two register sets and its peeled last one or two blocks (and the
# tiles that load one block at a time).  Rows per block: 2 (bf16 H = 4096),
# 64 (bf16 H = 128), 1 (bf16 H = 8192), 4 (fp32 H = 896), 1 (bf16 H = 16384).
MULTI_BLOCK = [(synth.BF16, 1026, 4096), (synth.BF16, 1539, 4096), (synth.BF16, 2559, 4096),
               (synth.BF16, 32868, 128), (synth.BF16, 775, 8192), (synth.F32, 2053, 896),
               (synth.BF16, 513, 16384)]


@pytest.mark.parametrize("mode", ["saved_rstd", "recompute", "dres"])
@pytest.mark.parametrize("dtype,rows,H", MULTI_BLOCK)
def test_bwd_multi_block(dtype, rows, H, mode):
    wl, x, w, dy, _, dres = _inputs(rows, H, dtype, seed=11 * rows + H, outliers=0.01)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    _, r64 = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    rstd32 = round_f32(r64)
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    rstd_d = torch.from_numpy(rstd32.astype(np.float32)).to(DEV) if mode != "recompute" else None
    dres_d = to_dev(dres, dtype) if mode == "dres" else None
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_bwd(dyd, xd, wd, rstd_d, dres_d, dx, dw, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps,
                                  rstd=None if mode == "recompute" else rstd32,
                                  dres=synth.to_f64(dres, dtype) if mode == "dres" else None)
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


# Narrow rows in such numbers that the forward's grid (at least 4 KB of x
# per workgroup, at least 2048 workgroups) gives every workgroup two or three
# row blocks: the loop that loads the next block while finishing the current
# one, and its last, partly filled block.
MANY_BLOCKS = [(synth.BF16, 3_000_017, 1), (synth.BF16, 1_500_007, 2),
               (synth.BF16, 700_001, 4), (synth.F32, 2_000_003, 1)]


@pytest.mark.parametrize("dtype,rows,H", MANY_BLOCKS)
def test_fwd_several_blocks_per_workgroup(dtype, rows, H):
    wl, x, w, _, res, _ = _inputs(rows, H, dtype, seed=rows % 1000 + H)
    xd, rd, wd = to_dev(x, dtype), to_dev(res, dtype), to_dev(w, dtype)
    y = _empty(rows, H, dtype)
    rstd = torch.full((rows,), float("nan"), device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
    h, y2 = _empty(rows, H, dtype), _empty(rows, H, dtype)
    rstd2 = torch.full((rows,), float("nan"), device=DEV)
    B.rmsnorm_residual_fwd(xd, rd, wd, h, y2, rstd2, wl.eps)
    torch.cuda.synchronize()
    x64, w64 = synth.to_f64(x, dtype), synth.to_f64(w, dtype)
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)
    kind = oracle.H_BF16 if dtype == synth.BF16 else oracle.H_F32
    ho, yo2, ro2 = oracle.rmsnorm_residual_fwd(x64, synth.to_f64(res, dtype), w64, wl.eps, kind)
    assert np.array_equal(f64(h), ho), "h must be bit-exact"
    assert_output("y", f64(y2), yo2, dtype)
    assert_rstd(f64(rstd2), ro2)


# The backward's workspace comes from the caller uninitialised.  Whatever it
# holds (here every float of it NaN, +inf or -inf) must not reach dw, also
# through the rows past the end of a partly filled last row block; nor may r
# recomputed at eps = 0, which is infinite for such rows' zero inputs.  Each
# shape leaves at least one workgroup with a partly filled last block.
STALE = [(synth.BF16, 300, 128), (synth.BF16, 3, 4096), (synth.BF16, 1539, 4096),
         (synth.BF16, 33, 896), (synth.F32, 2053, 896), (synth.BF16, 7, 500),
         (synth.F32, 5, 4095), (synth.BF16, 775, 8192), (synth.BF16, 19, 32768)]


@pytest.mark.parametrize("fill", ["nan", "inf", "-inf"])
@pytest.mark.parametrize("mode", ["saved_rstd", "recompute_eps0", "dres"])
@pytest.mark.parametrize("dtype,rows,H", STALE)
def test_bwd_ignores_stale_workspace(dtype, rows, H, mode, fill):
    eps = 0.0 if mode == "recompute_eps0" else 1e-6
    wl, x, w, dy, _, dres = _inputs(rows, H, dtype, seed=13 * rows + H)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    _, r64 = oracle.rmsnorm_fwd(x64, w64, eps)
    rstd32 = round_f32(r64)
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    saved = mode != "recompute_eps0"
    rstd_d = torch.from_numpy(rstd32.astype(np.float32)).to(DEV) if saved else None
    dres_d = to_dev(dres, dtype) if mode == "dres" else None
    ws = _ws(rows, H, dtype)
    ws[: ws.numel() // 4 * 4].view(torch.float32).fill_(float(fill))
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_bwd(dyd, xd, wd, rstd_d, dres_d, dx, dw, ws, eps)
    torch.cuda.synchronize()
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, eps, rstd=rstd32 if saved else None,
                                  dres=synth.to_f64(dres, dtype) if mode == "dres" else None)
    assert np.all(np.isfinite(f64(dw))), "dw picked up a non-finite value"
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


def _degenerate_rows(H, dtype):
    """Rows the method treats specially: all zeros (y = 0, r = 1/sqrt(eps)),
    constant rows of either sign, a single non-zero element, tiny and large
    magnitudes (still inside the fp32 range of the squares)."""
    rng = np.random.default_rng(H)
    rows = [np.zeros(H), np.full(H, 3.0), np.full(H, -0.5), np.zeros(H),
            rng.standard_normal(H) * 1e-12, rng.standard_normal(H) * 1e9]
    rows[3][H // 3] = 5.0
    return synth.quantise(np.stack(rows).astype(np.float32), dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H", [128, 896, 4096, 8192])
def test_degenerate_rows(dtype, H):
    x = _degenerate_rows(H, dtype)
    rows = x.shape[0]
    wl, _, w, dy, *_ = _inputs(rows, H, dtype, seed=H + 3)
    eps = 1e-6
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    y, rstd = _empty(rows, H, dtype), torch.full((rows,), float("nan"), device=DEV)
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    yo, ro = oracle.rmsnorm_fwd(x64, w64, eps)
    r32, r32_d = oracle_stat(ro)
    B.rmsnorm_fwd(xd, wd, y, rstd, eps)
    B.rmsnorm_bwd(dyd, xd, wd, r32_d, None, dx, dw, _ws(rows, H, dtype), eps)
    torch.cuda.synchronize()
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)
    assert_rstd_rounded(f64(rstd), ro)
    assert np.all(f64(y)[0] == 0.0), "a zero row gives y = 0"
    assert f64(rstd)[0] == float(np.float32(1.0 / math.sqrt(eps))), "zero row: r = 1/sqrt(eps)"
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, eps, rstd=r32)
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


def _same_nonfinite(name, g, o):
    """g and o are NaN at the same places and equal (0 == -0) elsewhere."""
    assert np.array_equal(np.isnan(g), np.isnan(o)), f"{name}: NaN pattern differs from the oracle"
    fin = ~np.isnan(o)
    assert np.array_equal(g[fin], o[fin]), f"{name}: non-NaN values differ from the oracle"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H", [128, 896, 4096, 8192, 16384, 32768])
@pytest.mark.parametrize("saved", [True, False])
def test_nonfinite_inputs_stay_in_their_row(dtype, H, saved):
    """Rows are independent (P1 §4.1, §5.3), so a NaN or an infinity in x
    reaches only its own row of y, rstd and dx, with what the double-precision
    definition gives there: a NaN row is NaN throughout; a row holding one
    infinity has mean(x^2) = inf, so r = 0, y = w x r is 0 except NaN where x
    is infinite, and dx = r (w dy - x r^2 c) is NaN.  dw sums over every row,
    so it is NaN in every column.  Every finite row is checked as usual."""
    rows = 7
    wl, x, w, dy, *_ = _inputs(rows, H, dtype, seed=H + 17)
    x = synth.to_f64(x, dtype).astype(np.float32)
    x[1, H // 2] = np.nan
    x[3, H - 1] = np.inf
    x[5, 0] = -np.inf
    x = synth.quantise(x, dtype)
    bad, good = [1, 3, 5], [0, 2, 4, 6]
    eps = wl.eps
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    y, rstd = _empty(rows, H, dtype), torch.empty(rows, device=DEV)
    dx = _empty(rows, H, dtype)
    dw = torch.zeros(H, dtype=torch_dtype(dtype), device=DEV)
    yo, ro = oracle.rmsnorm_fwd(x64, w64, eps)
    r32, r32_d = oracle_stat(ro)
    B.rmsnorm_fwd(xd, wd, y, rstd, eps)
    B.rmsnorm_bwd(dyd, xd, wd, r32_d if saved else None, None, dx, dw, _ws(rows, H, dtype), eps)
    torch.cuda.synchronize()
    yg, rg, dxg, dwg = f64(y), f64(rstd), f64(dx), f64(dw)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, eps, rstd=r32 if saved else None)
    assert np.isnan(ro[1]) and ro[3] == 0.0 and ro[5] == 0.0, "oracle: r of the NaN and inf rows"
    assert np.isnan(rg[1]) and rg[3] == 0.0 and rg[5] == 0.0, f"rstd of the non-finite rows: {rg[bad]}"
    for i in bad:
        _same_nonfinite(f"y row {i}", yg[i], yo[i])
        _same_nonfinite(f"dx row {i}", dxg[i], dxo[i])
        assert np.isnan(dxg[i]).all(), f"dx row {i} should be NaN throughout"
    assert np.isnan(dwo).all() and np.isnan(dwg).all(), "dw should be NaN in every column"
    assert_output("y", yg[good], yo[good], dtype)
    assert_rstd_rounded(rg[good], ro[good])
    assert_output("dx", dxg[good], dxo[good], dtype)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", [(37, 128), (9, 896), (300, 4096), (5, 8192), (3, 16384),
                                    (2, 32768), (2, 65536), (1000, 77)])
def test_documented_aliasing(rows, H, dtype):
    """The aliasing the C header allows gives the same bits as separate
    buffers: h written over x or over res in the residual forward (an
    in-place residual update), and dx written over dy or over dres in the
    backward, on every kind of row kernel (register tiles, LDS-staged,
    row-in-LDS, streaming, scalar)."""
    wl, x, w, dy, res, dres = _inputs(rows, H, dtype, seed=rows + H + 29)
    xd, wd, dyd, rd, drd = (to_dev(a, dtype) for a in (x, w, dy, res, dres))
    eps = wl.eps
    h, y, rstd = _empty(rows, H, dtype), _empty(rows, H, dtype), torch.empty(rows, device=DEV)
    B.rmsnorm_residual_fwd(xd, rd, wd, h, y, rstd, eps)
    for over in ("x", "res"):
        xa, ra = xd.clone(), rd.clone()
        ya, ra_st = _empty(rows, H, dtype), torch.empty(rows, device=DEV)
        ha = xa if over == "x" else ra
        B.rmsnorm_residual_fwd(xa, ra, wd, ha, ya, ra_st, eps)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ha), _bits(h)), f"h over {over}"
        assert torch.equal(_bits(ya), _bits(y)) and torch.equal(ra_st, rstd), f"y, rstd (h over {over})"
    dx, dw = _empty(rows, H, dtype), torch.empty(H, dtype=torch_dtype(dtype), device=DEV)
    ws = _ws(rows, H, dtype)
    for saved in (rstd, None):
        B.rmsnorm_bwd(dyd, h, wd, saved, drd, dx, dw, ws, eps)
        for over in ("dy", "dres"):
            dya, dra = dyd.clone(), drd.clone()
            dwa = torch.empty_like(dw)
            dxa = dya if over == "dy" else dra
            B.rmsnorm_bwd(dya, h, wd, saved, dra, dxa, dwa, ws, eps)
            torch.cuda.synchronize()
            assert torch.equal(_bits(dxa), _bits(dx)), f"dx over {over} (rstd saved: {saved is not None})"
            assert torch.equal(_bits(dwa), _bits(dw)), f"dw (dx over {over})"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("H", [1, 7, 896, 4096])
def test_constant_rows_eps0_give_signed_w(dtype, H):
    """At eps = 0 a constant row x = c (c = +-2^k) has r = 1/|c| exactly and
    y = sign(c) w bit for bit."""
    cs = [1.0, -1.0, 8.0, -0.25, 2.0 ** -20, -(2.0 ** 30)]
    x = np.stack([np.full(H, c) for c in cs])
    x = synth.quantise(x.astype(np.float32), dtype)
    rows = len(cs)
    _, _, w, *_ = _inputs(rows, H, dtype, seed=H + 5)
    xd, wd = to_dev(x, dtype), to_dev(w, dtype)
    y, rstd = _empty(rows, H, dtype), torch.empty(rows, device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, 0.0)
    torch.cuda.synchronize()
    w64 = synth.to_f64(w, dtype)
    for i, c in enumerate(cs):
        assert f64(rstd)[i] == 1.0 / abs(c), (i, c)
        assert np.array_equal(f64(y)[i], math.copysign(1.0, c) * w64), (i, c)


def _random_case(k):
    """Seeded draw of a shape and kind: H across every tile class (and odd
    widths, which take the scalar path), rows from one to a few hundred."""
    rng = np.random.default_rng(9000 + k)
    dtype = DTYPES[k % 2]
    H = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, 1100)),
                        int(rng.integers(1100, 4200)), int(rng.integers(4200, 16385))]))
    if rng.random() < 0.6:          # mostly widths that allow 128-bit accesses
        H = max(8, H // 8 * 8)
    rows = int(rng.integers(1, max(2, min(400, 2_000_000 // H))))
    mode = ["saved_rstd", "recompute", "dres"][k % 3]
    return dtype, rows, H, mode


@pytest.mark.parametrize("k", range(60))
def test_random_shapes(k):
    """Forward (plain or residual) and backward on seeded random shapes,
    element by element against the oracle."""
    dtype, rows, H, mode = _random_case(k)
    wl, x, w, dy, res, dres = _inputs(rows, H, dtype, seed=100 + k, outliers=0.01)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    rstd = torch.full((rows,), float("nan"), device=DEV)
    if mode == "dres":
        rd = to_dev(res, dtype)
        h, y = _empty(rows, H, dtype), _empty(rows, H, dtype)
        B.rmsnorm_residual_fwd(xd, rd, wd, h, y, rstd, wl.eps)
        kind = oracle.H_BF16 if dtype == synth.BF16 else oracle.H_F32
        ho, yo, ro = oracle.rmsnorm_residual_fwd(x64, synth.to_f64(res, dtype), w64, wl.eps, kind)
        torch.cuda.synchronize()
        assert np.array_equal(f64(h), ho), "h must be bit-exact"
        xin, xin64 = h, ho
    else:
        y = _empty(rows, H, dtype)
        B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
        yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
        xin, xin64 = xd, x64
    torch.cuda.synchronize()
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)
    # The GPU backward chains the forward's rstd, which must be the oracle's
    # statistic bitwise; the oracle is given that statistic from its own r.
    assert_rstd_rounded(f64(rstd), ro)
    dres_d = to_dev(dres, dtype) if mode == "dres" else None
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_bwd(dyd, xin, wd, None if mode == "recompute" else rstd, dres_d, dx, dw,
                  _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    dxo, dwo = oracle.rmsnorm_bwd(dy64, xin64, w64, wl.eps,
                                  rstd=None if mode == "recompute" else round_f32(ro),
                                  dres=synth.to_f64(dres, dtype) if mode == "dres" else None)
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", [(64, 896), (33, 4096), (300, 128), (9, 8192)])
def test_chain_fwd_then_bwd(rows, H, dtype):
    """GPU forward's rstd fed to the GPU backward, against the oracle with r
    recomputed in double: rstd within 2e-6, then dx/dw to the same bars."""
    wl, x, w, dy, *_ = _inputs(rows, H, dtype, seed=rows + H)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    y, rstd = _empty(rows, H, dtype), torch.empty(rows, device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
    dx = _empty(rows, H, dtype)
    dw = torch.empty(H, dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_bwd(dyd, xd, wd, rstd, None, dx, dw, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    assert_rstd(f64(rstd), ro)
    # The GPU's rstd must be the fp32 rounding of the oracle's r on every row;
    # the chained backward then matches the oracle given that statistic.
    assert_rstd_rounded(f64(rstd), ro)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps, rstd=round_f32(ro))
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,H", [(1, 896), (3, 896), (2, 4096), (1, 7), (4, 100)])
@pytest.mark.parametrize("splits", [1, 2, 4, 8, 16, 64])
def test_splitrow(rows, H, dtype, splits):
    wl, x, w, *_ = _inputs(rows, H, dtype, seed=11 * H + rows)
    xd, wd = to_dev(x, dtype), to_dev(w, dtype)
    y = _empty(rows, H, dtype)
    rstd = torch.empty(rows, device=DEV)
    n = B.rmsnorm_splitrow_partials_count(rows, splits)
    # The partial buffer is larger than needed and poisoned: the merge must
    # read only its own `splits` entries per row.
    partials = torch.full((n + 64,), float("nan"), device=DEV)
    B.rmsnorm_fwd_splitrow(xd, wd, y, rstd, partials, splits, wl.eps)
    torch.cuda.synchronize()
    yo, ro = oracle.rmsnorm_fwd(synth.to_f64(x, dtype), synth.to_f64(w, dtype), wl.eps)
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)
    assert torch.isnan(partials[n:]).all()


@pytest.mark.parametrize("dtype", DTYPES)
def test_unaligned_pointers_use_scalar_path(dtype):
    """Row pointers off the 16-byte grid (one-element offset views)."""
    rows, H = 37, 1024
    wl, x, w, dy, *_ = _inputs(rows, H, dtype, seed=99)
    td = torch_dtype(dtype)

    def off(a):
        t = to_dev(a.reshape(-1), dtype)
        buf = torch.empty(t.numel() + 1, dtype=td, device=DEV)
        buf[1:].copy_(t)
        return buf[1:].view(a.shape)

    xd, wd, dyd = off(x), off(w), off(dy)
    ybuf = torch.full((rows * H + 1,), float("nan"), dtype=td, device=DEV)
    y = ybuf[1:].view(rows, H)
    rstd = torch.empty(rows, device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
    dxbuf = torch.full((rows * H + 1,), float("nan"), dtype=td, device=DEV)
    dx = dxbuf[1:].view(rows, H)
    dw = torch.empty(H, dtype=td, device=DEV)
    B.rmsnorm_bwd(dyd, xd, wd, rstd, None, dx, dw, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    assert_output("y", f64(y), yo, dtype)
    assert_rstd_rounded(f64(rstd), ro)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps, rstd=round_f32(ro))
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)
    assert torch.isnan(ybuf[0]) and torch.isnan(dxbuf[0])


def test_rows_zero():
    H = 256
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    y = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    B.rmsnorm_fwd(x, w, y, None, 1e-6)
    dw = torch.full((H,), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.rmsnorm_bwd(x, x, w, None, None, y, dw, None, 1e-6)
    torch.cuda.synchronize()
    assert (dw == 0).all()


# A partly filled last row block on every tile kind (rows per block 64, 8, 2,
# 1, 4) and the scalar path.
GUARD = [(synth.BF16, 129, 896), (synth.BF16, 300, 128), (synth.BF16, 3, 4096),
         (synth.BF16, 1539, 4096), (synth.BF16, 5, 8192), (synth.BF16, 7, 500),
         (synth.F32, 2053, 896), (synth.F32, 5, 4095), (synth.BF16, 9, 32768),
         (synth.F32, 5, 12289), (synth.BF16, 7, 16384), (synth.BF16, 3, 12000)]


@pytest.mark.parametrize("dtype,rows,H", GUARD)
def test_guard_bands_untouched(dtype, rows, H):
    """Outputs sit between sentinel bands; the kernels write every output
    element and nothing outside."""
    wl, x, w, dy, res, dres = _inputs(rows, H, dtype, seed=3)
    G = 4096
    td = torch_dtype(dtype)

    def banded(n):
        buf = torch.full((n + 2 * G,), 12345.0, dtype=td, device=DEV)
        buf[G:G + n] = float("nan")
        return buf, buf[G:G + n]

    xd, wd, dyd, rd, drd = (to_dev(a, dtype) for a in (x, w, dy, res, dres))
    hb, h = banded(rows * H)
    yb, y = banded(rows * H)
    dxb, dx = banded(rows * H)
    dwb, dw = banded(H)
    rb = torch.full((rows + 2 * G,), 777.0, device=DEV)
    rstd = rb[G:G + rows]
    y2b, y2 = banded(rows * H)
    dx2b, dx2 = banded(rows * H)
    dw2b, dw2 = banded(H)
    rb2 = torch.full((rows + 2 * G,), 777.0, device=DEV)
    rstd2 = rb2[G:G + rows]
    B.rmsnorm_residual_fwd(xd, rd, wd, h.view(rows, H), y.view(rows, H), rstd, wl.eps)
    B.rmsnorm_bwd(dyd, h.view(rows, H), wd, rstd, drd, dx.view(rows, H), dw, _ws(rows, H, dtype),
                  wl.eps)
    B.rmsnorm_fwd(xd, wd, y2.view(rows, H), rstd2, wl.eps)
    B.rmsnorm_bwd(dyd, xd, wd, rstd2, None, dx2.view(rows, H), dw2, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    for buf, n in ((hb, rows * H), (yb, rows * H), (dxb, rows * H), (dwb, H),
                   (y2b, rows * H), (dx2b, rows * H), (dw2b, H)):
        assert (buf[:G] == 12345.0).all() and (buf[G + n:] == 12345.0).all()
        assert not torch.isnan(buf[G:G + n]).any()
    for band, r in ((rb, rstd), (rb2, rstd2)):
        assert (band[:G] == 777.0).all() and (band[G + rows:] == 777.0).all()
        assert not torch.isnan(r).any()


@pytest.mark.parametrize("dtype,rows,H,mode", [
    (synth.BF16, 1000, 4096, "saved_rstd"), (synth.F32, 1000, 4096, "saved_rstd"),
    (synth.BF16, 2559, 4096, "dres"), (synth.BF16, 2559, 4096, "recompute"),
    (synth.BF16, 775, 8192, "saved_rstd"), (synth.BF16, 32868, 128, "dres")])
def test_deterministic(dtype, rows, H, mode):
    """Fixed reduction order: repeated calls give bitwise-identical results
    (shapes with one to five row blocks per workgroup, each backward kind)."""
    wl, x, w, dy, _, dres = _inputs(rows, H, dtype, seed=1)
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    drd = to_dev(dres, dtype) if mode == "dres" else None
    outs = []
    for _ in range(3):
        y, rstd = _empty(rows, H, dtype), torch.empty(rows, device=DEV)
        dx, dw = _empty(rows, H, dtype), torch.empty(H, dtype=torch_dtype(dtype), device=DEV)
        B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
        B.rmsnorm_bwd(dyd, xd, wd, None if mode == "recompute" else rstd, drd, dx, dw,
                      _ws(rows, H, dtype), wl.eps)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()
                     for t in (y, rstd, dx, dw)])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_two_pass_api_equals_bwd():
    rows, H, dtype = 300, 2048, synth.BF16
    wl, x, w, dy, *_ = _inputs(rows, H, dtype, seed=8)
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    dx1, dx2 = _empty(rows, H, dtype), _empty(rows, H, dtype)
    dw1 = torch.empty(H, dtype=torch.bfloat16, device=DEV)
    dw2 = torch.empty(H, dtype=torch.bfloat16, device=DEV)
    ws = _ws(rows, H, dtype)
    B.rmsnorm_bwd(dyd, xd, wd, None, None, dx1, dw1, ws, wl.eps)
    B.rmsnorm_bwd_rows(dyd, xd, wd, None, None, dx2, ws, wl.eps)
    B.rmsnorm_bwd_dw_reduce(ws, dw2, rows)
    torch.cuda.synchronize()
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dw1.view(torch.int16), dw2.view(torch.int16))


def test_errors_are_reported():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(x)
    with pytest.raises(B.RMSNormError) as e:
        B.rmsnorm_fwd(x, w, y, None, eps=-1.0)
    assert e.value.status == B.EINVAL
    ws = torch.empty(1, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.RMSNormError) as e:
        B.rmsnorm_bwd(x, x, w, None, None, y, torch.empty(64, dtype=torch.bfloat16, device=DEV),
                      ws, 1e-6)
    assert e.value.status == B.EWORKSPACE


@pytest.mark.parametrize("rows,H", [(300, 896), (1539, 4096)])
def test_graph_capture_replays_match_eager(rows, H):
    """Every entry point records into a HIP graph (no allocation, no sync, no
    memset inside); replays, with eager work and synchronisation in between,
    reproduce the eager results bit for bit (one row block per backward
    workgroup, and three to four), and the replayed outputs match the oracle."""
    dtype = synth.BF16
    wl, x, w, dy, res, dres = _inputs(rows, H, dtype, seed=77)
    xd, wd, dyd, rd, drd = (to_dev(a, dtype) for a in (x, w, dy, res, dres))
    td = torch.bfloat16
    out = {k: torch.empty((rows, H), dtype=td, device=DEV) for k in ("y", "h", "y2", "dx", "ys")}
    rstd = torch.empty(rows, device=DEV)
    rstd2 = torch.empty(rows, device=DEV)
    dw = torch.empty(H, dtype=td, device=DEV)
    ws = _ws(rows, H, dtype)
    parts = torch.empty(B.rmsnorm_splitrow_partials_count(rows, 8), device=DEV)

    def work():
        B.rmsnorm_fwd(xd, wd, out["y"], rstd, wl.eps)
        B.rmsnorm_residual_fwd(xd, rd, wd, out["h"], out["y2"], rstd2, wl.eps)
        B.rmsnorm_bwd(dyd, out["h"], wd, rstd2, drd, out["dx"], dw, ws, wl.eps)
        B.rmsnorm_fwd_splitrow(xd, wd, out["ys"], None, parts, 8, wl.eps)

    work()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    ref_dw, ref_r = dw.clone(), rstd.clone()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        work()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        work()
    for rep in range(3):
        for v in list(out.values()) + [dw, rstd]:
            v.fill_(float("nan"))      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k].view(torch.int16), ref[k].view(torch.int16)), (rep, k)
        assert torch.equal(dw.view(torch.int16), ref_dw.view(torch.int16))
        assert torch.equal(rstd, ref_r)
    # The last replay's outputs against the oracle (not only against eager).
    x64, w64, dy64, r64, dr64 = (synth.to_f64(a, dtype) for a in (x, w, dy, res, dres))
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    assert_output("y (replay)", f64(out["y"]), yo, dtype)
    assert_rstd_rounded(f64(rstd), ro)
    assert_output("y splitrow (replay)", f64(out["ys"]), yo, dtype)
    ho, yo2, ro2 = oracle.rmsnorm_residual_fwd(x64, r64, w64, wl.eps, oracle.H_BF16)
    assert np.array_equal(f64(out["h"]), ho), "h (replay) must be bit-exact"
    assert_output("y residual (replay)", f64(out["y2"]), yo2, dtype)
    assert_rstd_rounded(f64(rstd2), ro2)
    dho, dwo = oracle.rmsnorm_bwd(dy64, ho, w64, wl.eps, rstd=round_f32(ro2), dres=dr64)
    assert_output("dh (replay)", f64(out["dx"]), dho, dtype)
    assert_dw(f64(dw), dwo, dtype)


@pytest.mark.parametrize("dtype,rows,H", [(synth.BF16, 3, 32768), (synth.BF16, 2, 65536),
                                          (synth.BF16, 2, 30000), (synth.F32, 2, 16384),
                                          (synth.F32, 1, 65536)])
def test_widest_rows(dtype, rows, H):
    """The widest rows, up to H = RMSNORM_MAX_H, through the residual pair."""
    wl, x, w, dy, res, dres = _inputs(rows, H, dtype, seed=H + rows)
    xd, wd, dyd, rd, drd = (to_dev(a, dtype) for a in (x, w, dy, res, dres))
    h, y, dx = _empty(rows, H, dtype), _empty(rows, H, dtype), _empty(rows, H, dtype)
    rstd = torch.empty(rows, device=DEV)
    dw = torch.empty(H, dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_residual_fwd(xd, rd, wd, h, y, rstd, wl.eps)
    B.rmsnorm_bwd(dyd, h, wd, rstd, drd, dx, dw, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    kind = oracle.H_BF16 if dtype == synth.BF16 else oracle.H_F32
    ho, yo, ro = oracle.rmsnorm_residual_fwd(synth.to_f64(x, dtype), synth.to_f64(res, dtype),
                                             synth.to_f64(w, dtype), wl.eps, kind)
    assert np.array_equal(f64(h), ho)
    assert_output("y", f64(y), yo, dtype)
    assert_rstd(f64(rstd), ro)
    assert_rstd_rounded(f64(rstd), ro)
    dxo, dwo = oracle.rmsnorm_bwd(synth.to_f64(dy, dtype), ho, synth.to_f64(w, dtype), wl.eps,
                                  rstd=round_f32(ro), dres=synth.to_f64(dres, dtype))
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


# Rows served by the streaming backward (the geometry's 1024-lane teams with
# 4 or more chunks per lane: 1024-lane workgroups with 4 slices, 512-lane
# ones with 16 and 32, the scalar path, partly filled last slices) and by the
# LDS-staged kernel below them (1024 x 2; 8200 bf16 and 4100 fp32 leave all
# but one lane's second chunk past H), with enough rows that every workgroup
# takes several (the next row loads during the current one).
WIDE = [(synth.BF16, 37, 16384), (synth.BF16, 19, 32768), (synth.BF16, 9, 65536),
        (synth.BF16, 23, 12000), (synth.F32, 21, 8192), (synth.F32, 11, 32768),
        (synth.F32, 5, 65536), (synth.BF16, 13, 1500), (synth.BF16, 7, 9001),
        (synth.F32, 6, 16383), (synth.BF16, 29, 8200), (synth.F32, 17, 4100)]


# More rows than workgroups, so that each workgroup of the LDS-staged and
# streaming kernels carries its prefetch across several rows.
WIDE_MULTI = [(synth.BF16, 600, 12288), (synth.BF16, 520, 24576), (synth.BF16, 300, 65536),
              (synth.F32, 530, 6144), (synth.F32, 300, 20000), (synth.F32, 290, 12288),
              (synth.BF16, 270, 20000), (synth.BF16, 3, 32760), (synth.F32, 260, 16384)]


@pytest.mark.parametrize("mode", ["saved_rstd", "recompute", "dres", "dres_recompute"])
@pytest.mark.parametrize("dtype,rows,H", WIDE + WIDE_MULTI)
def test_bwd_wide_rows(dtype, rows, H, mode):
    """Every wide-row kernel in each of its four builds: with or without a
    residual-stream gradient, saved or recomputed rstd."""
    recompute = mode.endswith("recompute")
    with_dres = mode.startswith("dres")
    wl, x, w, dy, _, dres = _inputs(rows, H, dtype, seed=17 * rows + H, outliers=0.01)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    _, r64 = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    rstd32 = round_f32(r64)
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    rstd_d = None if recompute else torch.from_numpy(rstd32.astype(np.float32)).to(DEV)
    dres_d = to_dev(dres, dtype) if with_dres else None
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_bwd(dyd, xd, wd, rstd_d, dres_d, dx, dw, _ws(rows, H, dtype), wl.eps)
    torch.cuda.synchronize()
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps,
                                  rstd=None if recompute else rstd32,
                                  dres=synth.to_f64(dres, dtype) if with_dres else None)
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)


def test_scalar_path_width_limit():
    """Rows that miss the 128-bit path are limited to RMSNORM_MAX_H_SCALAR;
    wider ones are refused, not mis-computed."""
    H = B.MAX_H_SCALAR + 1                     # odd: scalar accesses
    x = torch.zeros((2, H), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(x)
    with pytest.raises(B.RMSNormError) as e:
        B.rmsnorm_fwd(x, w, y, None, 1e-6)
    assert e.value.status == B.EUNSUPPORTED
    H = B.MAX_H_SCALAR - 1                     # largest odd width that is served
    wl, xa, wa, *_ = _inputs(2, H, synth.BF16, seed=5)
    xd, wd = to_dev(xa, synth.BF16), to_dev(wa, synth.BF16)
    y = _empty(2, H, synth.BF16)
    B.rmsnorm_fwd(xd, wd, y, None, wl.eps)
    torch.cuda.synchronize()
    yo, _ = oracle.rmsnorm_fwd(synth.to_f64(xa, synth.BF16), synth.to_f64(wa, synth.BF16), wl.eps)
    assert_output("y", f64(y), yo, synth.BF16)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale_exp", [-70, 70, 100])
@pytest.mark.parametrize("H", [128, 896, 4096, 8192])
def test_extreme_magnitudes(dtype, scale_exp, H):
    """Rows of x ~ N(0,1) * 2^k with k = -70, 70, 100 at eps = 0: squares and
    w*dy*x products far outside fp32's range of exact products are formed in
    fp64, so y, rstd, dx and dw still match the oracle to the usual bars (a
    product formed in fp32 would overflow to inf, giving NaN, at 2^70 and
    lose bits to underflow at 2^-70)."""
    rows = 9
    wl, x, w, dy, *_ = _inputs(rows, H, dtype, seed=H + 100 + scale_exp)
    x = synth.quantise((synth.to_f64(x, dtype) * 2.0 ** scale_exp).astype(np.float32), dtype)
    x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (x, w, dy))
    assert np.all(np.isfinite(x64)) and np.max(np.abs(x64)) > 0
    eps = 0.0
    yo, ro = oracle.rmsnorm_fwd(x64, w64, eps)
    r32, r32_d = oracle_stat(ro)
    xd, wd, dyd = to_dev(x, dtype), to_dev(w, dtype), to_dev(dy, dtype)
    y, rstd = _empty(rows, H, dtype), torch.full((rows,), float("nan"), device=DEV)
    dx = _empty(rows, H, dtype)
    dw = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    dxq = _empty(rows, H, dtype)
    dwq = torch.full((H,), float("nan"), dtype=torch_dtype(dtype), device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, eps)
    B.rmsnorm_bwd(dyd, xd, wd, r32_d, None, dx, dw, _ws(rows, H, dtype), eps)
    B.rmsnorm_bwd(dyd, xd, wd, None, None, dxq, dwq, _ws(rows, H, dtype), eps)
    torch.cuda.synchronize()
    assert_output("y", f64(y), yo, dtype)
    assert_rstd_rounded(f64(rstd), ro)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, eps, rstd=r32)
    assert_output("dx", f64(dx), dxo, dtype)
    assert_dw(f64(dw), dwo, dtype)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, eps, rstd=None)
    assert_output("dx (recompute)", f64(dxq), dxo, dtype)
    assert_dw(f64(dwq), dwo, dtype)
