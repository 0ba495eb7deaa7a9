"""GPU parity at the workloads' full sizes, through the same entry points and
launch configuration the benchmark times, against the double-precision
oracle on every element (the C oracle runs these sizes in seconds).

Workloads (synthetic, seeded; see bwd_rmsnorm_fwd_amd/synth.py):
  c1 fp32 64x896, c2 bf16 4096x4096 with outlier feature columns,
  c3 bf16 decode 1x896 (split-row with 4/8/16 splits and unsplit),
  c4 bf16 residual 16384x4096 (+ its backward with dres),
  c5a bf16 262144x128, c5b bf16 8192x8192.
"""
import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_fwd_amd import binding as B
from bwd_rmsnorm_fwd_amd import synth
from _gpu_util import (DEV, assert_dw, assert_output, assert_rstd, assert_rstd_rounded, f64,
                       oracle_stat, to_dev, torch_dtype)

pytestmark = pytest.mark.gpu

TRAIN = ["c1_f32_64x896", "c2_bf16_4096x4096", "c5a_bf16_262144x128", "c5b_bf16_8192x8192"]


def _ws(rows, H, dtype):
    code = B.F32 if dtype == synth.F32 else B.BF16
    return torch.empty(max(B.rmsnorm_bwd_workspace_bytes(rows, H, code), 16), dtype=torch.uint8,
                       device=DEV)


@pytest.mark.parametrize("name", TRAIN)
def test_workload_fwd_bwd(name):
    """Forward, then the backward three ways: given the oracle's statistic
    (fp32 rounding of its double r, the same input on both sides), chained
    from the GPU forward's saved rstd (which must equal that statistic on
    every row, so the chained dx and dw must equal the first ones bitwise),
    and recomputing r from x (the oracle recomputes it in double)."""
    wl = synth.WORKLOADS[name]
    rows, H, dt = wl.rows, wl.H, wl.dtype
    print(f"[full] {name}: rows={rows} H={H} dtype={dt}", flush=True)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    xd, wd, dyd = to_dev(x, dt), to_dev(w, dt), to_dev(dy, dt)
    td = torch_dtype(dt)
    y = torch.empty((rows, H), dtype=td, device=DEV)
    rstd = torch.empty(rows, device=DEV)
    B.rmsnorm_fwd(xd, wd, y, rstd, wl.eps)
    torch.cuda.synchronize()
    x64, w64, dy64 = (synth.to_f64(a, dt) for a in (x, w, dy))
    del x, dy
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    e_y = assert_output("y", f64(y), yo, dt)
    del yo, y
    e_r = assert_rstd(f64(rstd), ro)
    assert_rstd_rounded(f64(rstd), ro)
    r32, r32_d = oracle_stat(ro)

    def bwd(stat):
        dx = torch.empty((rows, H), dtype=td, device=DEV)
        dw = torch.empty(H, dtype=td, device=DEV)
        ws = _ws(rows, H, dt)
        B.rmsnorm_bwd_rows(dyd, xd, wd, stat, None, dx, ws, wl.eps)
        B.rmsnorm_bwd_dw_reduce(ws, dw, rows)
        torch.cuda.synchronize()
        return dx, dw

    dx, dw = bwd(r32_d)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps, rstd=r32)
    e_dx = assert_output("dx", f64(dx), dxo, dt)
    e_dw = assert_dw(f64(dw), dwo, dt)
    del dxo
    dxc, dwc = bwd(rstd)
    assert torch.equal(dxc.view(torch.int16 if dt == synth.BF16 else torch.int32),
                       dx.view(torch.int16 if dt == synth.BF16 else torch.int32)), "chained dx"
    assert torch.equal(dwc, dw), "chained dw"
    del dxc, dwc, dx, dw
    dxq, dwq = bwd(None)
    dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps, rstd=None)
    e_dxq = assert_output("dx (recompute)", f64(dxq), dxo, dt)
    e_dwq = assert_dw(f64(dwq), dwo, dt)
    print(f"[full] {name}: y {e_y:.3g}  rstd {e_r:.3g}  dx {e_dx:.3g}  dw {e_dw:.3g}  "
          f"recompute: dx {e_dxq:.3g}  dw {e_dwq:.3g}", flush=True)


def test_workload_residual_fwd_bwd():
    """Residual forward, then its backward with dres given the oracle's
    statistic, chained from the GPU forward's rstd (bitwise the same), and
    recomputing r from h."""
    wl = synth.WORKLOADS["c4_bf16_residual_16384x4096"]
    rows, H, dt = wl.rows, wl.H, wl.dtype
    print(f"[full] {wl.name}: rows={rows} H={H}", flush=True)
    x, res, w, dy, dres = wl.x(), wl.res(), wl.w(), wl.dy(), wl.dres()
    xd, rd, wd, dyd, drd = (to_dev(a, dt) for a in (x, res, w, dy, dres))
    td = torch_dtype(dt)
    h = torch.empty((rows, H), dtype=td, device=DEV)
    y = torch.empty((rows, H), dtype=td, device=DEV)
    rstd = torch.empty(rows, device=DEV)
    B.rmsnorm_residual_fwd(xd, rd, wd, h, y, rstd, wl.eps)
    torch.cuda.synchronize()
    del xd, rd
    ho, yo, ro = oracle.rmsnorm_residual_fwd(synth.to_f64(x, dt), synth.to_f64(res, dt),
                                             synth.to_f64(w, dt), wl.eps, oracle.H_BF16)
    del x, res
    assert np.array_equal(f64(h), ho), "h must be bit-exact"
    e_y = assert_output("y", f64(y), yo, dt)
    del yo, y
    e_r = assert_rstd(f64(rstd), ro)
    assert_rstd_rounded(f64(rstd), ro)
    r32, r32_d = oracle_stat(ro)
    dy64, w64, dres64 = synth.to_f64(dy, dt), synth.to_f64(w, dt), synth.to_f64(dres, dt)

    def bwd(stat):
        dh = torch.empty((rows, H), dtype=td, device=DEV)
        dw = torch.empty(H, dtype=td, device=DEV)
        B.rmsnorm_bwd(dyd, h, wd, stat, drd, dh, dw, _ws(rows, H, dt), wl.eps)
        torch.cuda.synchronize()
        return dh, dw

    dh, dw = bwd(r32_d)
    dho, dwo = oracle.rmsnorm_bwd(dy64, ho, w64, wl.eps, rstd=r32, dres=dres64)
    e_dh = assert_output("dh", f64(dh), dho, dt)
    e_dw = assert_dw(f64(dw), dwo, dt)
    del dho
    dhc, dwc = bwd(rstd)
    assert torch.equal(dhc.view(torch.int16), dh.view(torch.int16)), "chained dh"
    assert torch.equal(dwc.view(torch.int16), dw.view(torch.int16)), "chained dw"
    del dhc, dwc, dh, dw
    dhq, dwq = bwd(None)
    dho, dwo = oracle.rmsnorm_bwd(dy64, ho, w64, wl.eps, rstd=None, dres=dres64)
    e_dhq = assert_output("dh (recompute)", f64(dhq), dho, dt)
    e_dwq = assert_dw(f64(dwq), dwo, dt)
    print(f"[full] {wl.name}: y {e_y:.3g}  rstd {e_r:.3g}  dh {e_dh:.3g}  dw {e_dw:.3g}  "
          f"recompute: dh {e_dhq:.3g}  dw {e_dwq:.3g}", flush=True)


@pytest.mark.parametrize("splits", [1, 4, 8, 16])
def test_workload_decode_splitrow(splits):
    wl = synth.WORKLOADS["c3_bf16_decode_1x896"]
    rows, H, dt = wl.rows, wl.H, wl.dtype
    x, w = wl.x(), wl.w()
    xd, wd = to_dev(x, dt), to_dev(w, dt)
    y = torch.empty((rows, H), dtype=torch_dtype(dt), device=DEV)
    rstd = torch.empty(rows, device=DEV)
    partials = torch.full((B.rmsnorm_splitrow_partials_count(rows, splits) + 16,), float("nan"),
                          device=DEV)
    B.rmsnorm_fwd_splitrow(xd, wd, y, rstd, partials, splits, wl.eps)
    y_plain = torch.empty_like(y)
    B.rmsnorm_fwd(xd, wd, y_plain, None, wl.eps)
    torch.cuda.synchronize()
    yo, ro = oracle.rmsnorm_fwd(synth.to_f64(x, dt), synth.to_f64(w, dt), wl.eps)
    assert_output("y", f64(y), yo, dt)
    assert_rstd(f64(rstd), ro)
    # Split and unsplit agree to within one bf16 ulp of each other.
    assert np.max(np.abs(f64(y) - f64(y_plain))) <= np.max(np.abs(yo)) * 2.0 ** -7


# (block rows P, H): the register tile, the LDS-staged and the row-in-LDS
# backward kernels.  P divides neither the row count nor 2^31 / H.
BEYOND = [(4099, 4096), (1031, 12288), (257, 32768)]


@pytest.mark.parametrize("P,H", BEYOND)
def test_beyond_2_31_elements(P, H):
    """Tensors of just over 2^31 bf16 elements (2^31 / H + 3 rows): every
    offset past 2^31 elements (2^32 bytes) must reach its own row.  The input
    is a seeded block of P rows tiled on the device; 2^31 / H rows is not a
    multiple of P, so an index that wrapped would read a row holding other
    values.  The block's outputs are checked against the oracle, and every
    row of the large run must equal its block row bitwise (row outputs do not
    depend on the rest of the batch); dw is checked against the oracle with dy
    scaled by each block row's repeat count (dw is linear in dy)."""
    rows = (1 << 31) // H + 3
    dt = synth.BF16
    wl = synth.small_case(P, H, dt, seed=31, residual=True)
    x, w, dy, res = wl.x(), wl.w(), wl.dy(), wl.res()
    print(f"[full] beyond 2^31 elements: rows={rows} H={H} bf16 (block of {P} rows)", flush=True)
    xs, ws_, dys, rs_ = to_dev(x, dt), to_dev(w, dt), to_dev(dy, dt), to_dev(res, dt)
    reps = (rows + P - 1) // P

    def tile(t):
        return t.repeat(reps, 1)[:rows].contiguous()

    def run(xd, dyd, rd, n, stat=None):
        """Forward, backward (given `stat`, else chained from this forward's
        rstd) and residual forward on n rows."""
        y = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
        rstd = torch.empty(n, device=DEV)
        dx = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
        dw = torch.empty(H, dtype=torch.bfloat16, device=DEV)
        B.rmsnorm_fwd(xd, ws_, y, rstd, wl.eps)
        B.rmsnorm_bwd(dyd, xd, ws_, rstd if stat is None else stat, None, dx, dw, _ws(n, H, dt),
                      wl.eps)
        h = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
        yr = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
        rr = torch.empty(n, device=DEV)
        B.rmsnorm_residual_fwd(xd, rd, ws_, h, yr, rr, wl.eps)
        torch.cuda.synchronize()
        return y, rstd, dx, dw, h, yr, rr

    # The block: its backward takes the oracle's statistic (fp32 of its r),
    # which the block's forward must reproduce bitwise.
    x64, w64, dy64 = (synth.to_f64(a, dt) for a in (x, w, dy))
    yo, ro = oracle.rmsnorm_fwd(x64, w64, wl.eps)
    r32, r32_d = oracle_stat(ro)
    small = run(xs, dys, rs_, P, stat=r32_d)
    assert_output("y", f64(small[0]), yo, dt)
    assert_rstd(f64(small[1]), ro)
    assert_rstd_rounded(f64(small[1]), ro)
    dxo, _ = oracle.rmsnorm_bwd(dy64, x64, w64, wl.eps, rstd=r32)
    assert_output("dx", f64(small[2]), dxo, dt)
    ho, _, _ = oracle.rmsnorm_residual_fwd(x64, synth.to_f64(res, dt), w64, wl.eps, oracle.H_BF16)
    assert np.array_equal(f64(small[4]), ho), "h must be bit-exact"

    # The large run chains its own forward's rstd into its backward; its rows
    # must equal the block's (whose rstd is the oracle's statistic) bitwise.
    xb, dyb, rb = tile(xs), tile(dys), tile(rs_)
    assert xb.numel() > (1 << 31)
    big = run(xb, dyb, rb, rows)
    del xb, dyb, rb
    full = (rows // P) * P
    for name, b, s in zip(("y", "rstd", "dx", "dw", "h", "y(res)", "rstd(res)"), big, small):
        if name == "dw":
            continue
        bb = b[:full].reshape(rows // P, P, *b.shape[1:])
        assert torch.equal(bb, s.unsqueeze(0).expand_as(bb)), f"{name}: rows differ from the block"
        assert torch.equal(b[full:], s[:rows - full]), f"{name}: tail rows differ from the block"
    count = np.full(P, rows // P, dtype=np.float64)
    count[:rows - full] += 1
    _, dwo = oracle.rmsnorm_bwd(dy64 * count[:, None], x64, w64, wl.eps, rstd=r32)
    e_dw = assert_dw(f64(big[3]), dwo, dt)
    print(f"[full] beyond 2^31 elements: rows match the block bitwise, dw {e_dw:.3g}", flush=True)
