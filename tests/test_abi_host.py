"""C ABI checks that need no GPU: the library loads, exports every function
include/*.h declares, and rejects bad arguments before touching the device.

The validation checks pass pseudo-pointers that must be rejected before any
launch.  So that a change in the order of the checks could never launch a
kernel on an unmapped address, each of them runs in a child process that
sees no GPU (HIP_VISIBLE_DEVICES and ROCR_VISIBLE_DEVICES name no device):
there a launch that slipped through returns an error instead of running.
The child first confirms that HIP reports no device, else it refuses to run."""
import ctypes
import glob
import os
import re
import subprocess
import sys

import pytest

from bwd_rmsnorm_fwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b((?:rmsnorm|decode_gemv)_\w+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_residual_fwd", "rmsnorm_fwd_splitrow",
               "rmsnorm_bwd_workspace_bytes", "rmsnorm_status_str"):
        assert fn in names, names


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for fn in declared_functions():
        assert hasattr(L, fn), f"{fn} declared in include/ but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT ((?:rmsnorm|decode_gemv)_\w+)", out))
    assert set(declared_functions()) == exported, exported ^ set(declared_functions())


def test_header_compiles_as_c():
    """The header is plain C (extern "C" guarded) and compiles alone."""
    src = '#include "rmsnorm.h"\nint main(void){return (int)RMSNORM_OK;}\n'
    r = subprocess.run(["gcc", "-x", "c", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    for code in range(7):
        assert B.status_str(code) != "unknown status"
    assert B.status_str(99) == "unknown status"


def _fwd(*a):
    return B.lib().rmsnorm_fwd(*a)


MIS = ctypes.c_void_p(0x1001)  # misaligned pseudo-pointer: rejected before any launch


def _check_fwd_validation():
    nul = None
    stream = None
    assert _fwd(nul, nul, nul, nul, 4, 64, 1e-6, B.BF16, stream) == B.EINVAL       # null pointers
    assert _fwd(MIS, MIS, MIS, nul, 4, 64, 1e-6, 7, stream) == B.EINVAL            # bad dtype
    assert _fwd(MIS, MIS, MIS, nul, -1, 64, 1e-6, B.BF16, stream) == B.EINVAL      # rows < 0
    assert _fwd(MIS, MIS, MIS, nul, 4, 0, 1e-6, B.BF16, stream) == B.EINVAL        # H < 1
    assert _fwd(MIS, MIS, MIS, nul, 4, 64, -1e-6, B.BF16, stream) == B.EINVAL      # eps < 0
    assert _fwd(MIS, MIS, MIS, nul, 4, 64, float("nan"), B.BF16, stream) == B.EINVAL
    assert _fwd(MIS, MIS, MIS, nul, 4, 64, float("inf"), B.BF16, stream) == B.EINVAL
    assert _fwd(MIS, MIS, MIS, nul, 4, B.MAX_H + 1, 1e-6, B.BF16, stream) == B.EUNSUPPORTED
    assert _fwd(MIS, MIS, MIS, nul, 4, 64, 1e-6, B.BF16, stream) == B.EALIGN       # odd address
    assert _fwd(MIS, MIS, MIS, nul, 0, 64, 1e-6, B.BF16, stream) == B.OK           # rows = 0: no-op


def _check_bwd_validation_and_workspace():
    L = B.lib()
    need = L.rmsnorm_bwd_workspace_bytes(4096, 4096, B.BF16)
    assert need > 0 and need % 16 == 0
    assert L.rmsnorm_bwd_workspace_bytes(0, 4096, B.BF16) == 0
    assert L.rmsnorm_bwd_workspace_bytes(-1, 4096, B.BF16) == 0
    assert L.rmsnorm_bwd_workspace_bytes(10, 0, B.BF16) == 0
    A = ctypes.c_void_p(0x10000)  # aligned pseudo-pointer, never dereferenced here
    # Workspace too small is caught before any launch.
    st = L.rmsnorm_bwd(A, A, A, None, None, A, A, A, need - 1, 4096, 4096, 1e-6, B.BF16, None)
    assert st == B.EWORKSPACE
    st = L.rmsnorm_bwd(A, A, A, None, None, A, A, None, 0, 4096, 4096, 1e-6, B.BF16, None)
    assert st == B.EWORKSPACE
    st = L.rmsnorm_bwd(A, A, A, None, None, A, None, A, need, 4096, 4096, 1e-6, B.BF16, None)
    assert st == B.EINVAL                                                   # dw missing
    st = L.rmsnorm_bwd(A, None, A, None, None, A, A, A, need, 4096, 4096, 1e-6, B.BF16, None)
    assert st == B.EINVAL                                                   # x missing
    st = L.rmsnorm_bwd(A, A, A, None, MIS, A, A, A, need, 4096, 4096, 1e-6, B.BF16, None)
    assert st == B.EALIGN                                                   # misaligned dres
    st = L.rmsnorm_bwd_rows(A, A, A, None, None, A, A, need, 0, 4096, 1e-6, B.BF16, None)
    assert st == B.EINVAL                                                   # rows pass needs rows
    # Workspace size is a pure function of the shape: monotone in rows, capped.
    sizes = [L.rmsnorm_bwd_workspace_bytes(r, 4096, B.BF16) for r in (1, 8, 64, 1024, 1 << 20)]
    assert sizes == sorted(sizes) and sizes[-1] == sizes[-2]


def _check_splitrow_validation():
    L = B.lib()
    A = ctypes.c_void_p(0x10000)
    assert L.rmsnorm_splitrow_partials_count(1, 4) == 4
    assert L.rmsnorm_splitrow_partials_count(3, 16) == 48
    assert L.rmsnorm_splitrow_partials_count(1, 0) == 0
    assert L.rmsnorm_splitrow_partials_count(1, B.MAX_SPLITS + 1) == 0
    f = L.rmsnorm_fwd_splitrow
    assert f(A, A, A, None, A, 4, 1, 896, 1e-6, 0, B.BF16, None) == B.EINVAL        # splits = 0
    assert f(A, A, A, None, A, 4, 1, 896, 1e-6, 65, B.BF16, None) == B.EINVAL       # > max
    assert f(A, A, A, None, A, 3, 1, 896, 1e-6, 4, B.BF16, None) == B.EWORKSPACE    # too few
    assert f(A, A, A, None, None, 4, 1, 896, 1e-6, 4, B.BF16, None) == B.EWORKSPACE
    assert f(A, A, A, None, A, 4, 0, 896, 1e-6, 4, B.BF16, None) == B.EINVAL        # rows = 0


def _check_gemv_validation():
    L = B.lib()
    A = ctypes.c_void_p(0x10000)
    assert L.decode_gemv_partials_count(1024, 4) == 4096
    assert L.decode_gemv_partials_count(1024, 1) == 0
    assert L.decode_gemv_partials_count(0, 4) == 0
    f = L.decode_gemv_splitk
    assert f(A, A, A, A, 4096, 1024, 896, 0, B.BF16, None) == B.EINVAL        # splits = 0
    assert f(A, A, A, A, 4096, 1024, 896, 65, B.BF16, None) == B.EINVAL       # > max
    assert f(A, A, A, A, 4095, 1024, 896, 4, B.BF16, None) == B.EWORKSPACE    # too few partials
    assert f(A, A, A, None, 0, 1024, 896, 4, B.BF16, None) == B.EWORKSPACE
    assert f(A, None, A, None, 0, 1024, 896, 1, B.BF16, None) == B.EINVAL     # x missing
    assert f(A, A, A, None, 0, 0, 896, 1, B.BF16, None) == B.EINVAL           # N = 0
    assert f(MIS, A, A, None, 0, 8, 896, 1, B.BF16, None) == B.EALIGN


def _dry(fn, *args):
    B.rmsnorm_set_dry_run(True)
    try:
        st = fn(*args)
        return st, [l for l in B.rmsnorm_dry_run_report().splitlines() if l]
    finally:
        B.rmsnorm_set_dry_run(False)


def _check_dispatch_of_workloads():
    """Which kernels each configured workload launches (dry run: validated as
    usual, recorded instead of launched), and the launch shapes that carry the
    design: one team per row, several rows per wavefront for narrow rows, at
    most one backward workgroup per CU, S split workgroups for decode."""
    L = B.lib()
    A = ctypes.c_void_p(0x10000)
    eps = ctypes.c_float(1e-6)

    def fwd(rows, H, dt):
        return _dry(L.rmsnorm_fwd, A, A, A, A, rows, H, eps, dt, None)

    def bwd(rows, H, dt, dres=None, rstd=A):
        need = L.rmsnorm_bwd_workspace_bytes(rows, H, dt)
        return _dry(L.rmsnorm_bwd, A, A, A, rstd, dres, A, A, A, need, rows, H, eps, dt, None)

    def grid(line):
        return int(line.split("grid=")[1].split("x")[0])

    # c1 fp32 64 x 896; c2 bf16 4096 x 4096; c5a 262144 x 128; c5b 8192 x 8192.
    for rows, H, dt, t in ((64, 896, B.F32, "float, 4"), (4096, 4096, B.BF16, "unsigned short, 8"),
                           (262144, 128, B.BF16, "unsigned short, 8"),
                           (8192, 8192, B.BF16, "unsigned short, 8")):
        st, f = fwd(rows, H, dt)
        assert st == B.OK and len(f) == 1 and f[0].startswith(f"rms::fwd_kernel<{t},"), f
        st, b = bwd(rows, H, dt)
        assert st == B.OK and len(b) == 2, b
        assert "bwd_rows" in b[0] and f"<{t}," in b[0] and "dw_reduce_kernel" in b[1], b
        assert grid(b[0]) <= 256, b                      # at most one workgroup per CU
    # Narrow rows: a 16-lane team per 128-wide bf16 row, 4 rows per wavefront.
    assert "rms::fwd_kernel<unsigned short, 8, 16, 1," in fwd(262144, 128, B.BF16)[1][0]
    assert "rms::bwd_rows_kernel<unsigned short, 8, 16, 1," in bwd(262144, 128, B.BF16)[1][0]
    # c4: residual forward and the backward with dres.
    st, f = _dry(L.rmsnorm_residual_fwd, A, A, A, A, A, A, 16384, 4096, eps, B.BF16, None)
    assert st == B.OK and len(f) == 1 and f[0].startswith("rms::fwd_kernel<unsigned short, 8,")
    assert f[0].split(" grid=")[0].endswith("true>"), f
    st, b = bwd(16384, 4096, B.BF16, dres=A)
    assert st == B.OK and b[0].split(" grid=")[0].endswith("true>"), b
    # c3 decode: S split workgroups, then one partial-reduce workgroup.
    for S in (1, 4, 8, 16):
        st, d = _dry(L.rmsnorm_fwd_splitrow, A, A, A, A, A, S, 1, 896, eps, S, B.BF16, None)
        assert st == B.OK and len(d) == 2, d
        assert d[0].startswith("rms::split_sumsq_kernel") and f"grid=1x{S}x1" in d[0], d
        assert d[1].startswith("rms::split_finalize_kernel") and "grid=1x1x1" in d[1], d
    # q_proj GEMV 1024 x 896: one kernel unsplit; partials + splitk_reduce split.
    for S in (1, 4, 8, 16):
        n = L.decode_gemv_partials_count(1024, S)
        st, g = _dry(L.decode_gemv_splitk, A, A, A, A if S > 1 else None, n, 1024, 896, S, B.BF16,
                     None)
        assert st == B.OK and len(g) == (1 if S == 1 else 2), g
        assert g[0].startswith("rms::gemv_splitk_kernel<unsigned short,"), g
        if S > 1:
            assert g[1].startswith("rms::splitk_reduce_kernel<unsigned short>"), g
    # Wide rows: the LDS-staged, row-in-LDS and streaming backward kernels.
    assert "bwd_rows_staged_kernel" in bwd(2730, 12288, B.BF16)[1][0]
    assert "bwd_rows_ldsrow_kernel" in bwd(2048, 32768, B.BF16)[1][0]
    assert "bwd_rows_wide_kernel" in bwd(2048, 32768, B.BF16, dres=A)[1][0]
    assert "bwd_rows_wide_kernel" in bwd(1024, 65536, B.BF16)[1][0]
    # rows = 0: nothing to launch for the forward; the backward still writes dw.
    assert fwd(0, 4096, B.BF16) == (B.OK, [])
    # A call that fails validation records nothing.
    st, d = _dry(L.rmsnorm_fwd, A, A, A, A, 4, 64, ctypes.c_float(-1.0), B.BF16, None)
    assert st == B.EINVAL and d == []


def _check_bench_stream_validation():
    """The benchmark's plain-stream helper refuses arguments outside its
    limits before any HIP call."""
    sys.path.insert(0, ROOT)
    import bench
    SL = bench.stream_lib()
    assert SL is not None, "libbench_stream.so is not built"
    A = ctypes.c_void_p(0x10000)
    f = SL.bench_stream
    assert f(0, 1, 0, A, None, None, A, None, 8192, None) == 1        # no read stream
    assert f(4, 1, 0, A, A, A, A, None, 8192, None) == 1               # more than 3 reads
    assert f(1, 3, 0, A, None, None, A, A, 8192, None) == 1            # more than 2 writes
    assert f(1, 1, 2, A, None, None, A, None, 8192, None) == 1         # no such access kind
    assert f(1, 1, 1, A, None, None, A, None, 8191, None) == 1         # not whole 8 KB blocks
    assert f(1, 1, 0, A, None, None, A, None, 0, None) == 1
    assert f(2, 1, 0, A, None, None, A, None, 8192, None) == 1         # second read missing
    assert f(1, 2, 1, A, None, None, A, None, 8192, None) == 1         # second write missing
    assert f(1, 1, 0, MIS, None, None, A, None, 8192, None) == 1       # misaligned


HIDDEN_ENV = {"HIP_VISIBLE_DEVICES": "-1", "ROCR_VISIBLE_DEVICES": "-1", "CUDA_VISIBLE_DEVICES": "-1"}

CHILD = r"""
import ctypes, os, sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(-1)
st = hip.hipGetDeviceCount(ctypes.byref(n))
if st == 0 and n.value > 0:
    print("a GPU is visible to the validation child", file=sys.stderr)
    sys.exit(3)
import test_abi_host as t
getattr(t, {fn!r})()
print("ok")
"""


@pytest.mark.parametrize("check", ["_check_fwd_validation", "_check_bwd_validation_and_workspace",
                                   "_check_splitrow_validation", "_check_gemv_validation",
                                   "_check_dispatch_of_workloads",
                                   "_check_bench_stream_validation"])
def test_validation_without_a_device(check):
    env = dict(os.environ, **HIDDEN_ENV)
    code = CHILD.format(tests=os.path.dirname(os.path.abspath(__file__)), root=ROOT, fn=check)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout, r.stderr)


def test_binding_rejects_mismatched_tensors():
    """The Python binding refuses host tensors and wrong sizes before any call."""
    import torch
    x = torch.zeros((4, 8), dtype=torch.bfloat16)
    w = torch.zeros(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.rmsnorm_fwd(x, w, x.clone(), None)      # host tensors are refused


def test_bench_refuses_multi_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_byte_formulas():
    sys.path.insert(0, ROOT)
    import bench
    # rows * (2 H e + 4) + H e for the forward of the bf16 4096 x 4096 workload.
    assert bench.fwd_bytes(4096, 4096, 2) == 67_133_440
    assert bench.bwd_bytes(4096, 4096, 2) == 100_696_064
    assert bench.fwd_bytes(16384, 4096, 2, residual=True) == 536_944_640
    assert bench.bwd_bytes(16384, 4096, 2, dres=True) == 536_952_832
    assert bench.fwd_bytes(262144, 128, 2) == 135_266_560
    assert bench.bwd_bytes(8192, 8192, 2) == 402_718_720
    assert bench.fwd_bytes(64, 896, 4) == 462_592


def test_bench_cold_rotation():
    """The number of rotating buffer sets per workload: the other sets'
    forwards read at least 2.5 x the 256 MB Infinity Cache in between."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.cold_sets(16384, 4096, 2, residual=True) == 4
    assert bench.cold_sets(8192, 8192, 2) == 6
    assert bench.cold_sets(262144, 128, 2) == 11
    assert bench.cold_sets(4096, 4096, 2) == 21
    assert bench.cold_sets(64, 896, 4) == bench.MAX_SETS
    for rows, H, e, res in ((16384, 4096, 2, True), (8192, 8192, 2, False), (4096, 4096, 2, False)):
        k = bench.cold_sets(rows, H, e, res)
        read = rows * H * e * (2 if res else 1)
        assert (k - 1) * read >= bench.COLD_BYTES > (k - 2) * read


def test_bench_roofline_choice():
    """The roofline kernel is the longer of the forward and the row pass; the
    row pass counts as the smaller of its own burst and its (row pass, dw
    reduce) pair burst."""
    sys.path.insert(0, ROOT)
    import bench
    base = {"names": [["fwd_k"], ["rows_k"], ["red_k"]], "fwd_bytes": 10, "rows_bytes": 20}
    # Row pass slower alone than with its reduce: the pair's figure is used.
    r = dict(base, fwd_us=86.0, rows_us=95.0, bwd_us=88.0)
    assert bench.pick_roofline(r) == ("rows_k", 88.0, 20, "burst of (row pass, dw reduce) pairs, "
                                      "the reduce included", 88.0)
    # The row pass alone is the smaller figure and still longer than the forward.
    r = dict(base, fwd_us=86.0, rows_us=87.0, bwd_us=89.5)
    assert bench.pick_roofline(r)[:4] == ("rows_k", 87.0, 20, "burst of itself")
    # The forward is the longer kernel.
    r = dict(base, fwd_us=86.5, rows_us=86.2, bwd_us=88.9)
    assert bench.pick_roofline(r) == ("fwd_k", 86.5, 10, "burst of itself", 86.2)
