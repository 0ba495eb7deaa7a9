"""The backward entry point that allocates nothing (rmsnorm_bwd_noalloc),
called through the C ABI, against rmsnorm_bwd on the same inputs: dx and dw
must be bitwise equal (same kernels, same reduction order), on two calls in
a row, the second with a smaller input that reuses the same scratch; plus a
third call on the oracle's inputs against the oracle, and the refusal of a
shape that needs more scratch than the library holds, and the call recorded
under HIP graph capture."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from bwd_rmsnorm_fwd_amd import binding as B
from bwd_rmsnorm_fwd_amd import synth
from _gpu_util import DEV, assert_dw, assert_output, f64, oracle_stat, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def _case(rows, H, dtype, seed, dres):
    wl = synth.small_case(rows, H, dtype, seed=seed, outlier_frac=0.01)
    x, w, dy = wl.x(), wl.w(), wl.dy()
    _, ro = oracle.rmsnorm_fwd(synth.to_f64(x, dtype), synth.to_f64(w, dtype), wl.eps)
    r32, r32_d = oracle_stat(ro)
    d = {"wl": wl, "x": x, "w": w, "dy": dy, "r32": r32, "rstd": r32_d,
         "xd": to_dev(x, dtype), "wd": to_dev(w, dtype), "dyd": to_dev(dy, dtype),
         "dres": wl.dres() if dres else None}
    d["dresd"] = to_dev(d["dres"], dtype) if dres else None
    return d


def _noalloc(c, dtype, out=None):
    rows, H = c["xd"].shape
    td = torch_dtype(dtype)
    if out is None:
        out = (torch.full((rows, H), float("nan"), dtype=td, device=DEV),
               torch.full((H,), float("nan"), dtype=td, device=DEV))
    dx, dw = out
    L = B.lib()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = L.rmsnorm_bwd_noalloc(p(c["dyd"]), p(c["xd"]), p(c["wd"]), p(c["rstd"]), p(c["dresd"]),
                               p(dx), p(dw), rows, H, ctypes.c_float(c["wl"].eps),
                               B.F32 if dtype == synth.F32 else B.BF16,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == B.OK, B.status_str(st)
    return dx, dw


def _with_workspace(c, dtype):
    rows, H = c["xd"].shape
    td = torch_dtype(dtype)
    dx = torch.full((rows, H), float("nan"), dtype=td, device=DEV)
    dw = torch.full((H,), float("nan"), dtype=td, device=DEV)
    code = B.F32 if dtype == synth.F32 else B.BF16
    ws = torch.empty(max(B.lib().rmsnorm_bwd_workspace_bytes(rows, H, code), 16), dtype=torch.uint8,
                     device=DEV)
    B.rmsnorm_bwd(c["dyd"], c["xd"], c["wd"], c["rstd"], c["dresd"], dx, dw, ws, c["wl"].eps)
    return dx, dw


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dtype,big,small,dres", [
    (synth.BF16, (4096, 4096), (300, 896), False),
    (synth.BF16, (2048, 8192), (77, 4096), True),
    (synth.F32, (1024, 2048), (64, 896), False),
    (synth.BF16, (1030, 16384), (5, 129), True),
])
def test_noalloc_equals_bwd_twice(dtype, big, small, dres):
    print(f"[noalloc] {dtype} {big} then {small} dres={dres}", flush=True)
    for k, (rows, H) in enumerate((big, small)):
        c = _case(rows, H, dtype, seed=40 + k + rows % 97, dres=dres)
        dx_a, dw_a = _noalloc(c, dtype)
        torch.cuda.synchronize()
        dx_b, dw_b = _with_workspace(c, dtype)
        torch.cuda.synchronize()
        assert torch.equal(_bits(dx_a), _bits(dx_b)), (k, rows, H, "dx")
        assert torch.equal(_bits(dw_a), _bits(dw_b)), (k, rows, H, "dw")
        x64, w64, dy64 = (synth.to_f64(a, dtype) for a in (c["x"], c["w"], c["dy"]))
        dxo, dwo = oracle.rmsnorm_bwd(dy64, x64, w64, c["wl"].eps, rstd=c["r32"],
                                      dres=synth.to_f64(c["dres"], dtype) if dres else None)
        assert_output("dx", f64(dx_a), dxo, dtype)
        assert_dw(f64(dw_a), dwo, dtype)


def test_noalloc_recompute_and_refusal():
    c = _case(513, 4096, synth.BF16, seed=9, dres=False)
    c["rstd"] = None
    dx_a, dw_a = _noalloc(c, synth.BF16)
    dx_b, dw_b = _with_workspace(c, synth.BF16)
    torch.cuda.synchronize()
    assert torch.equal(_bits(dx_a), _bits(dx_b)) and torch.equal(_bits(dw_a), _bits(dw_b))
    # A shape whose partial rows exceed the scratch is refused before any
    # launch (asked in dry-run mode, so that nothing could launch regardless).
    L = B.lib()
    rows, H = 4096, 32768
    assert L.rmsnorm_bwd_workspace_bytes(rows, H, B.BF16) > B.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(0x10000)
    B.rmsnorm_set_dry_run(True)
    try:
        st = L.rmsnorm_bwd_noalloc(p, p, p, None, None, p, p, rows, H, ctypes.c_float(1e-6),
                                   B.BF16, None)
        assert B.rmsnorm_dry_run_report() == ""
    finally:
        B.rmsnorm_set_dry_run(False)
    assert st == B.ESCRATCH, B.status_str(st)


def test_noalloc_in_a_captured_graph():
    """Recorded under HIP graph capture (one of the callers the entry point is
    for), the call replays to the eager call's dx and dw bit for bit, also
    when an eager call of another shape has used the scratch in between."""
    dtype = synth.BF16
    c = _case(2048, 4096, dtype, seed=61, dres=True)
    other = _case(300, 896, dtype, seed=62, dres=False)
    dx_e, dw_e = _noalloc(c, dtype)
    torch.cuda.synchronize()
    rows, H = c["xd"].shape
    td = torch_dtype(dtype)
    dx = torch.empty((rows, H), dtype=td, device=DEV)
    dw = torch.empty((H,), dtype=td, device=DEV)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _noalloc(c, dtype, out=(dx, dw))
    torch.cuda.current_stream().wait_stream(s)
    for k in range(3):
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        _noalloc(other, dtype)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(dx), _bits(dx_e)), (k, "dx")
        assert torch.equal(_bits(dw), _bits(dw_e)), (k, "dw")
