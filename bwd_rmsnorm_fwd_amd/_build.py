"""Build librmsnorm_mi355x.so from csrc/ with hipcc for gfx950 (in-tree).

Each translation unit is compiled to an object in parallel, then linked into
one shared library next to this file.  Extra -D definitions (kernel tuning
constants) can be passed through ``defines``.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "librmsnorm_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["rmsnorm_api.hip", "rmsnorm_fwd.hip", "rmsnorm_bwd.hip", "rmsnorm_bwd_wide.hip",
           "rmsnorm_split.hip",
           "decode_gemv.hip", "decode_gemv_api.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    # Keep packed fp32 instructions out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(out_path: str = LIB_PATH, defines=(), build_dir: str | None = None, jobs: int = 8,
          verbose: bool = False) -> str:
    build_dir = build_dir or os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stdout.strip() or r.stderr.strip()):
            print(r.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out_path)
    build_bench_loops()
    build_bench_stream()
    return out_path


def resource_usage(src: str, defines=()) -> dict:
    """Per-kernel register, scratch and LDS use of one source file for gfx950,
    from the compiler's kernel resource-usage remarks (a device-only compile,
    no object kept).  Returns {mangled kernel name: {field: int}} with the
    fields TotalSGPRs, VGPRs, AGPRs, ScratchSize, Occupancy, SGPRsSpill,
    VGPRsSpill, LDSSize."""
    import re
    import tempfile
    dflags = [f"-D{d}" for d in defines]
    with tempfile.TemporaryDirectory() as td:
        cmd = [HIPCC, *FLAGS, *dflags, "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
               "-c", os.path.join(CSRC, src), "-o", os.path.join(td, "k.o")]
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    out: dict = {}
    cur = None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).replace(" ", "")] = int(m.group(2))
    return out


BENCH_LOOPS_SRC = os.path.join(PKG, "bench_loops.cpp")
BENCH_LOOPS_PATH = os.path.join(PKG, "libbench_loops.so")


def build_bench_loops(out_path: str = BENCH_LOOPS_PATH) -> str:
    """The benchmark's host launch loops (plain host C++, no device code)."""
    tmp = out_path + ".tmp"
    cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-shared", "-o", tmp, BENCH_LOOPS_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for bench_loops.cpp:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out_path)
    return out_path


BENCH_STREAM_SRC = os.path.join(PKG, "bench_stream.hip")
BENCH_STREAM_PATH = os.path.join(PKG, "libbench_stream.so")


def build_bench_stream(out_path: str = BENCH_STREAM_PATH) -> str:
    """The benchmark's plain-stream kernels (the ceiling figures), gfx950."""
    tmp = out_path + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", "-o", tmp, BENCH_STREAM_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for bench_stream.hip:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    import sys
    print(build(defines=sys.argv[1:], verbose=True))
