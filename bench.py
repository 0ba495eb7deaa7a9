#!/usr/bin/env python3
"""RMSNorm forward + backward throughput on one MI355X.

A step is one pass of the hot path over one batch: the fused residual-add +
RMSNorm forward (h and y written, rstd saved) then its backward (dh = dx +
dres and the dw partials, then the dw reduce pass) of the bf16 residual
workload rows = B*T = 4*4096 = 16384, H = 4096 (the largest configuration,
the shape of the pages' own forward benchmark), through the library's C ABI.
Inputs are resident in HBM before timing; buffer sets rotate so that each
kernel's inputs are out of the 256 MB Infinity Cache.

Prints one JSON line.  `value` is achieved HBM GB/s over the whole step,
counting the algorithmic bytes only (residual fwd: x, res, w read, h, y,
rstd written; bwd: dy, dres, h, w, rstd read, dh, dw written), by wall clock
over the timed steps.  `roofline` is for the step's dominant kernel, timed
with HIP events around a burst of its back-to-back launches before the
steps (the row pass also in a burst of row pass + dw reduce pairs), on the
stream it runs on; its name comes from the library's dry-run report.  `stream_ceiling` times plain streams of the same reads and writes
(bench_stream.hip: loads and stores only) on the same cold rotation, so each
kernel can be set against what merely moving its bytes takes.  `configs`
gives fwd and bwd µs (median and P95) / GB/s / % of 8 TB/s for every other
configuration, with its stream ceilings and a warm-buffer figure (not HBM),
and µs per call for decode (plain, C loop, HIP graph) and the split-K q_proj.
`cpu_baseline` times the double-precision oracle on the host, on one thread
and on all the cores this process may use.

--suite FILE also measures every workload in detail (median and P95, wide
rows, warm cache) and writes one JSON object per measurement to FILE.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of MI355X peak) + µs/call, RMSNorm fwd and bwd"
PEAK_GBS = 8000.0          # MI355X HBM3E
# Input bytes read by other calls between two uses of one buffer set: 2.5 x
# the 256 MB Infinity Cache.  Measured on the bf16 forwards with cached
# loads: with less, a call still finds part of its inputs there (8192 x 8192
# with 134 MB read in between: 86.5% of 8 TB/s; with 402 MB or more: 74%;
# 4096 x 4096 with 235 MB read in between: 73.7%, with 369 MB: 62.6%).
# Nontemporal loads do not allocate there (the backward's times do not
# depend on the number of sets), but the rule does not rely on it.
COLD_BYTES = 640 << 20
MAX_SETS = 64


# ---------------------------------------------------------------- algorithmic bytes

def fwd_bytes(rows, H, e, residual=False):
    """x (+res) read, y (+h) written, rstd written, w read once."""
    per_row = (4 if residual else 2) * H * e + 4
    return rows * per_row + H * e


def bwd_rows_bytes(rows, H, e, dres=False):
    """Row pass: dy, x (+dres) read, rstd read, dx written, w read once."""
    per_row = (4 if dres else 3) * H * e + 4
    return rows * per_row + H * e


def bwd_bytes(rows, H, e, dres=False):
    """Whole backward: the row pass plus dw written."""
    return bwd_rows_bytes(rows, H, e, dres) + H * e


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bwd_rmsnorm_fwd_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- device plumbing

def cold_sets(rows, H, e, residual=False):
    """Buffer sets to rotate so that the other sets' forwards read at least
    COLD_BYTES between two uses of one set (at least 2, at most MAX_SETS)."""
    read = rows * H * e * (2 if residual else 1)
    return min(MAX_SETS, max(2, math.ceil(COLD_BYTES / read) + 1))


class Sets:
    """K rotating buffer sets of one workload, filled with its seeded inputs.
    K is chosen so that between two uses of one set the other sets' calls of
    the kernel that reads least (the forward: x, and res) read at least
    COLD_BYTES: no call finds its inputs in the Infinity Cache.  (At most
    MAX_SETS: the smallest workload is launch-bound either way.)"""

    def __init__(self, wl, k=None, residual=False, dres=False):
        import numpy as np
        import torch
        from bwd_rmsnorm_fwd_amd import binding as B
        from bwd_rmsnorm_fwd_amd import synth

        self.wl = wl
        rows, H = wl.rows, wl.H
        self.e = 4 if wl.dtype == synth.F32 else 2
        td = torch.float32 if wl.dtype == synth.F32 else torch.bfloat16
        self.code = B.F32 if wl.dtype == synth.F32 else B.BF16

        def dev(a):
            if wl.dtype == synth.BF16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(td).cuda()
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()

        x, w, dy = dev(wl.x()), dev(wl.w()), dev(wl.dy())
        res = dev(wl.res()) if residual else None
        dres_t = dev(wl.dres()) if dres else None
        ws_bytes = max(B.rmsnorm_bwd_workspace_bytes(rows, H, self.code), 16)
        self.k = k or cold_sets(rows, H, self.e, residual)
        self.sets = []
        for _ in range(self.k):
            s = {
                "x": x.clone(), "w": w, "dy": dy.clone(),
                "y": torch.empty((rows, H), dtype=td, device="cuda"),
                "rstd": torch.empty(rows, dtype=torch.float32, device="cuda"),
                "dx": torch.empty((rows, H), dtype=td, device="cuda"),
                "dw": torch.empty(H, dtype=td, device="cuda"),
                "ws": torch.empty(ws_bytes, dtype=torch.uint8, device="cuda"),
            }
            if residual:
                s["res"] = res.clone()
                s["h"] = torch.empty((rows, H), dtype=td, device="cuda")
            if dres:
                s["dres"] = dres_t.clone()
            self.sets.append(s)
        self.ws_bytes = ws_bytes
        torch.cuda.synchronize()


class Calls:
    """Pre-marshalled C-ABI calls (pointers and sizes bound once) so that the
    host enqueues faster than the GPU drains."""

    def __init__(self, sets: Sets, stream):
        from bwd_rmsnorm_fwd_amd import binding as B
        self.L = B.lib()
        wl = sets.wl
        self.rows, self.H, self.eps, self.code = wl.rows, wl.H, ctypes.c_float(wl.eps), sets.code
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        self.sets = sets

    @staticmethod
    def p(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    def fwd(self, s):
        p = self.p
        return (self.L.rmsnorm_fwd, (p(s["x"]), p(s["w"]), p(s["y"]), p(s["rstd"]), self.rows, self.H,
                                     self.eps, self.code, self.stream))

    def residual_fwd(self, s):
        p = self.p
        return (self.L.rmsnorm_residual_fwd,
                (p(s["x"]), p(s["res"]), p(s["w"]), p(s["h"]), p(s["y"]), p(s["rstd"]), self.rows,
                 self.H, self.eps, self.code, self.stream))

    def bwd_rows(self, s, x_key="x", dres=False, saved_rstd=True):
        p = self.p
        return (self.L.rmsnorm_bwd_rows,
                (p(s["dy"]), p(s[x_key]), p(s["w"]), p(s["rstd"]) if saved_rstd else None,
                 p(s.get("dres")) if dres else None,
                 p(s["dx"]), p(s["ws"]), self.sets.ws_bytes, self.rows, self.H, self.eps, self.code,
                 self.stream))

    def bwd(self, s):
        p = self.p
        return (self.L.rmsnorm_bwd,
                (p(s["dy"]), p(s["x"]), p(s["w"]), p(s["rstd"]), None, p(s["dx"]), p(s["dw"]),
                 p(s["ws"]), self.sets.ws_bytes, self.rows, self.H, self.eps, self.code,
                 self.stream))

    def dw_reduce(self, s):
        p = self.p
        return (self.L.rmsnorm_bwd_dw_reduce,
                (p(s["ws"]), self.sets.ws_bytes, p(s["dw"]), self.rows, self.H, self.code,
                 self.stream))

    def splitrow(self, s, partials, splits):
        p = self.p
        return (self.L.rmsnorm_fwd_splitrow,
                (p(s["x"]), p(s["w"]), p(s["y"]), p(s["rstd"]), p(partials), partials.numel(),
                 self.rows, self.H, self.eps, splits, self.code, self.stream))


def c_loops():
    """The host launch-loop helper (bwd_rmsnorm_fwd_amd/bench_loops.cpp), or
    None when it has not been built."""
    path = os.path.join(ROOT, "bwd_rmsnorm_fwd_amd", "libbench_loops.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    L.bench_fwd_loop.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.bench_splitrow_loop.argtypes = [vp, i32, vp, vp, vp, vp, vp, sz, i64, i64, f32, i32, i32, vp]
    L.bench_gemv_loop.argtypes = [vp, i32, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    L.bench_bwd_loop.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f32, i32, vp]
    for f in (L.bench_fwd_loop, L.bench_splitrow_loop, L.bench_gemv_loop, L.bench_bwd_loop):
        f.restype = i32
    return L


def stream_lib():
    """The plain-stream kernels (bwd_rmsnorm_fwd_amd/bench_stream.hip), or
    None when they have not been built."""
    path = os.path.join(ROOT, "bwd_rmsnorm_fwd_amd", "libbench_stream.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bench_stream.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i64, vp]
    L.bench_stream.restype = i32
    return L


# Row tensors read and written by each kernel (w and rstd aside).
STREAM_PATTERN = {"fwd": (1, 1), "residual_fwd": (2, 2), "bwd_rows": (2, 1), "bwd_rows_dres": (3, 1)}


STREAM_ACCESS = ("global loads and stores", "buffer loads, device-scope buffer stores")


def stream_ceiling(SL, nr, nw, nbytes, stream, reps=13, burst=16):
    """A plain stream of `nr` reads and `nw` writes of `nbytes` each (rounded
    down to whole 8 KB blocks), timed like the configurations: `reps` bursts
    of `burst` launches over buffer sets rotating so that the other sets read
    at least COLD_BYTES between two uses of one set, for each access kind of
    bench_stream.hip (the two lead on different patterns); the faster one's
    median µs, GB/s and % of 8 TB/s over the bytes moved."""
    import torch
    nbytes = nbytes // 8192 * 8192
    if SL is None or nbytes == 0:
        return None
    k = min(MAX_SETS, max(2, math.ceil(COLD_BYTES / (nr * nbytes)) + 1))
    bufs = [[torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nr + nw)]
            for _ in range(k)]
    st = ctypes.c_void_p(stream.cuda_stream)
    best = None
    for kind, access in enumerate(STREAM_ACCESS):
        calls = []
        for b in bufs:
            ptr = [ctypes.c_void_p(t.data_ptr()) for t in b]
            ins = ptr[:nr] + [None] * (3 - nr)
            outs = ptr[nr:] + [None] * (2 - nw)
            calls.append(((SL.bench_stream, (nr, nw, kind, *ins, *outs, nbytes, st)),))
        (t,) = time_calls(calls, k, reps, 2 * k, stream, burst)
        us = statistics.median(t)
        if best is None or us < best[0]:
            best = (us, access)
    del bufs, calls
    torch.cuda.empty_cache()
    us, access = best
    gbs, pct = _pct((nr + nw) * nbytes, us)
    plural = lambda n, w: f"{n} {w}{'s' if n > 1 else ''}"
    return {"pattern": f"{plural(nr, 'read')} + {plural(nw, 'write')}", "access": access,
            "bytes_per_stream": nbytes, "buffer_sets": k, "us": round(us, 3), "GB_s": gbs,
            "pct_peak": pct}


def time_c_loop(loop, call, ncalls, stream):
    """µs per call of `call` (fn, args) made `ncalls` times back to back by a
    loop in C (loop(fn, n, *args)), bracketed by events on `stream`."""
    import torch
    fn, args = call
    fp = ctypes.cast(fn, ctypes.c_void_p)
    st = loop(fp, 200, *args)
    if st:
        raise RuntimeError(f"{fn.__name__}: status {st}")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    st = loop(fp, ncalls, *args)
    e1.record(stream)
    torch.cuda.synchronize()
    if st:
        raise RuntimeError(f"{fn.__name__}: status {st}")
    return e0.elapsed_time(e1) * 1e3 / ncalls


def run(call):
    fn, args = call
    st = fn(*args)
    if st != 0:
        from bwd_rmsnorm_fwd_amd import binding as B
        raise RuntimeError(f"{fn.__name__}: {B.status_str(st)}")


# ---------------------------------------------------------------- main benchmark

def step_plan(C, sets, residual=False):
    """Launch plan of one step per rotation slot: the forward of set i and the
    backward of set i + k/2 (whose forward ran k/2 steps earlier), so that no
    kernel reads data another kernel touched in the last ~0.5 GiB of traffic;
    the backward uses the statistic its set's forward saved."""
    k = sets.k
    plan = []
    for i in range(k):
        f = sets.sets[i]
        b = sets.sets[(i + k // 2) % k]
        if residual:
            plan.append((C.residual_fwd(f), C.bwd_rows(b, x_key="h", dres=True), C.dw_reduce(b)))
        else:
            plan.append((C.fwd(f), C.bwd_rows(b), C.dw_reduce(b)))
    return plan


HEADLINE = "c4_bf16_residual_16384x4096"


def kernel_names(C, calls):
    """Names of the kernels each call launches, from the library's dry run
    (the same entry point and arguments, nothing launched)."""
    from bwd_rmsnorm_fwd_amd import binding as B
    out = []
    for fn, args in calls:
        lines = B.launches_of(fn, *args)
        out.append([l.split(" grid=")[0] for l in lines])
    return out


def bench_step(steps, warmup, burst_min=200):
    """The headline step on the bf16 residual 16384 x 4096 workload.

    First the step's kernels in bursts: max(steps, burst_min) back-to-back
    launches over the rotating buffer sets, bracketed by HIP events recorded
    on the stream the kernels run on -- the forward alone, the backward row
    pass alone, and the row pass followed by its dw reduce; the average per
    launch is the kernel's duration plus the small dispatch gap between
    launches (the dw reduce is timed only with its row pass: a burst of the
    reduce alone would time the host's launch rate, its kernel being a few
    µs).  This also brings the GPU to its working clocks before the timed
    steps.  Then `warmup`
    untimed steps and `steps` timed steps (residual forward, backward row
    pass with the residual-stream gradient, dw reduce) back to back,
    bracketed by synchronisation, with nothing else enqueued between the
    launches; each step's backward works on a different buffer set than its
    forward (see step_plan), so both read their inputs from HBM."""
    import torch
    from bwd_rmsnorm_fwd_amd import synth

    wl = synth.WORKLOADS[HEADLINE]
    sets = Sets(wl, residual=True, dres=True)
    stream = torch.cuda.current_stream()
    C = Calls(sets, stream)
    plan = step_plan(C, sets, residual=True)
    names = kernel_names(C, plan[0])

    # Each kernel alone, event-bracketed bursts.
    nb = max(steps, burst_min)

    def burst(idx):
        for i in range(sets.k):
            for j in idx:
                run(plan[i][j])
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(nb):
            for j in idx:
                run(plan[i % sets.k][j])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / nb

    fwd_us, rows_us, bwd_us = burst((0,)), burst((1,)), burst((1, 2))

    for i in range(warmup):
        for c in plan[i % sets.k]:
            run(c)
    torch.cuda.synchronize()

    # The timed steps, wall clock.
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(steps):
        for c in plan[i % sets.k]:
            run(c)
    e_end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    span_ms = e_start.elapsed_time(e_end) / steps
    e = sets.e
    return {
        "wl": wl, "k": sets.k, "ms_step": ms_step, "span_ms": span_ms, "names": names,
        "burst": nb,
        "fwd_us": fwd_us, "rows_us": rows_us, "bwd_us": bwd_us,
        "fwd_bytes": fwd_bytes(wl.rows, wl.H, e, residual=True),
        "bwd_bytes": bwd_bytes(wl.rows, wl.H, e, dres=True),
        "rows_bytes": bwd_rows_bytes(wl.rows, wl.H, e, dres=True),
    }


def pick_roofline(r):
    """The dominant kernel of the headline step from its burst timings `r`
    (fwd_us, rows_us: bursts of each alone; bwd_us: burst of row pass + dw
    reduce pairs; names: kernel names per call; fwd_bytes, rows_bytes).  The
    row pass's figure is the smaller of its two bursts, each an upper bound
    on its duration.  Returns (name, µs, bytes, how it was timed, row-pass µs)."""
    rows_us, rows_basis = r["rows_us"], "burst of itself"
    if r["bwd_us"] < rows_us:
        rows_us, rows_basis = r["bwd_us"], "burst of (row pass, dw reduce) pairs, the reduce included"
    if r["fwd_us"] >= rows_us:
        return r["names"][0][0], r["fwd_us"], r["fwd_bytes"], "burst of itself", rows_us
    return r["names"][1][0], rows_us, r["rows_bytes"], rows_basis, rows_us


def _pct(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return round(gbs, 1), round(100 * gbs / PEAK_GBS, 2)


def _p95(us):
    v = sorted(us)
    return round(v[min(len(v) - 1, int(0.95 * len(v)))], 3)


def ceilings_of(wl, e, residual, fwd_gbs, rows_gbs, stream):
    """The plain streams of a workload's forward and backward row pass (same
    row tensors read and written, same size) and each kernel's GB/s as a
    fraction of its stream's."""
    SL = stream_lib()
    nbytes = wl.rows * wl.H * e
    cf = stream_ceiling(SL, *STREAM_PATTERN["residual_fwd" if residual else "fwd"], nbytes, stream)
    cb = stream_ceiling(SL, *STREAM_PATTERN["bwd_rows_dres" if residual else "bwd_rows"], nbytes,
                        stream)
    return {"stream_ceiling": {"fwd": cf, "bwd_rows": cb},
            "fwd_vs_stream": round(fwd_gbs / cf["GB_s"], 3) if cf else None,
            "bwd_rows_vs_stream": round(rows_gbs / cb["GB_s"], 3) if cb else None}


def config_table(reps=13, burst=16):
    """fwd / bwd µs per call (median of `reps` bursts of `burst` back-to-back
    launches on cold rotating buffers, events at the burst ends), GB/s and %
    of 8 TB/s over the algorithmic bytes, for every configuration; decode as
    µs per call over 10,000 back-to-back calls (Python loop, C loop, HIP
    graph replay); the split-K q_proj likewise."""
    import numpy as np
    import torch
    from bwd_rmsnorm_fwd_amd import binding as B
    from bwd_rmsnorm_fwd_amd import synth

    stream = torch.cuda.current_stream()
    out = {}
    for name in ("c1_f32_64x896", "c2_bf16_4096x4096", "c5a_bf16_262144x128",
                 "c5b_bf16_8192x8192", HEADLINE):
        wl = synth.WORKLOADS[name]
        res = wl.residual
        sets = Sets(wl, residual=res, dres=res)
        C = Calls(sets, stream)
        e = sets.e
        if res:
            f_calls = [(C.residual_fwd(s),) for s in sets.sets]
            b_calls = [(C.bwd_rows(s, x_key="h", dres=True), C.dw_reduce(s)) for s in sets.sets]
        else:
            f_calls = [(C.fwd(s),) for s in sets.sets]
            b_calls = [(C.bwd_rows(s), C.dw_reduce(s)) for s in sets.sets]
        (tf,) = time_calls(f_calls, sets.k, reps, 2 * sets.k, stream, burst)
        tr, tb = time_calls(b_calls, sets.k, reps, 2 * sets.k, stream, burst)
        (ts,) = time_calls(step_plan(C, sets, residual=res), sets.k, reps, 2 * sets.k, stream,
                           burst)[2:]
        # The same calls on one buffer set over and over (inputs partly or
        # wholly in the Infinity Cache): context only, not an HBM figure.
        (wf,) = time_calls(f_calls[:1], 1, reps, 2, stream, burst)
        wr, wb = time_calls(b_calls[:1], 1, reps, 2, stream, burst)
        fb = fwd_bytes(wl.rows, wl.H, e, residual=res)
        bb = bwd_bytes(wl.rows, wl.H, e, dres=res)
        rb = bwd_rows_bytes(wl.rows, wl.H, e, dres=res)
        med = lambda v: round(statistics.median(v), 3)
        d = {"rows": wl.rows, "H": wl.H, "dtype": wl.dtype, "residual": res,
             "fwd_us": med(tf), "bwd_rows_us": med(tr), "bwd_us": med(tb), "step_us": med(ts),
             "fwd_us_p95": _p95(tf), "bwd_rows_us_p95": _p95(tr), "bwd_us_p95": _p95(tb),
             "step_us_p95": _p95(ts), "fwd_bytes": fb, "bwd_bytes": bb}
        d["fwd_GB_s"], d["fwd_pct_peak"] = _pct(fb, d["fwd_us"])
        d["bwd_rows_GB_s"], d["bwd_rows_pct_peak"] = _pct(rb, d["bwd_rows_us"])
        d["bwd_GB_s"], d["bwd_pct_peak"] = _pct(bb, d["bwd_us"])
        d["step_GB_s"], d["step_pct_peak"] = _pct(fb + bb, d["step_us"])
        d["warm_same_buffers_not_hbm"] = {"fwd_us": med(wf), "bwd_rows_us": med(wr),
                                          "bwd_us": med(wb)}
        d["kernels"] = sorted({k for ks in kernel_names(C, step_plan(C, sets, residual=res)[0])
                               for k in ks})
        if name == "c1_f32_64x896":
            # Launch-bound: µs per call of the forward and of the whole
            # backward, also from a loop in C and replayed from HIP graphs.
            CL = c_loops()
            s0 = sets.sets[0]
            d["us_per_call"] = {
                "fwd": time_decode(lambda st: Calls(sets, st).fwd(s0), stream,
                                   CL.bench_fwd_loop if CL else None),
                "bwd": time_decode(lambda st: Calls(sets, st).bwd(s0), stream,
                                   CL.bench_bwd_loop if CL else None),
                "calls": 10000}
        del sets, C
        torch.cuda.empty_cache()
        d.update(ceilings_of(wl, e, res, d["fwd_GB_s"], d["bwd_rows_GB_s"], stream))
        out[name] = d

    # Decode rows = 1, H = 896: the one-wavefront row kernel and the split-row
    # path with S = 1, 4, 8, 16, each 10,000 calls back to back on one stream.
    CL = c_loops()
    wl = synth.WORKLOADS["c3_bf16_decode_1x896"]
    sets = Sets(wl, k=1)
    C = Calls(sets, stream)
    s = sets.sets[0]
    dec, dec_k = {}, {}
    for splits in (0, 1, 4, 8, 16):
        partials = torch.empty(max(splits, 1), dtype=torch.float32, device="cuda")

        def mk(st, partials=partials, splits=splits):
            Cs = Calls(sets, st)
            return Cs.fwd(s) if splits == 0 else Cs.splitrow(s, partials, splits)
        loop = None
        if CL is not None:
            loop = CL.bench_fwd_loop if splits == 0 else CL.bench_splitrow_loop
        label = "row_kernel" if splits == 0 else f"splitrow_S{splits}"
        dec[label] = time_decode(mk, stream, loop)
        dec_k[label] = kernel_names(C, [mk(stream)])[0]
    out["c3_bf16_decode_1x896"] = {"rows": 1, "H": wl.H, "dtype": wl.dtype,
                                   "us_per_call": dec, "calls": 10000, "kernels": dec_k}
    del sets, C

    gw = synth.GEMV_WORKLOADS["q_proj_bf16_1024x896"]
    A = torch.from_numpy(gw.A().view(np.int16)).view(torch.bfloat16).cuda()
    xv = torch.from_numpy(gw.x().view(np.int16)).view(torch.bfloat16).cuda()
    yv = torch.empty(gw.N, dtype=torch.bfloat16, device="cuda")
    L = B.lib()
    gq = {}
    for splits in gw.splits:
        parts = torch.empty(max(B.decode_gemv_partials_count(gw.N, splits), 1), device="cuda")

        def mk(st, parts=parts, splits=splits):
            return (L.decode_gemv_splitk,
                    (ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(xv.data_ptr()),
                     ctypes.c_void_p(yv.data_ptr()), ctypes.c_void_p(parts.data_ptr()),
                     parts.numel(), gw.N, gw.K, splits, B.BF16, ctypes.c_void_p(st.cuda_stream)))
        gq[f"S{splits}"] = time_decode(mk, stream, CL.bench_gemv_loop if CL else None)
    out["q_proj_bf16_1024x896"] = {"N": gw.N, "K": gw.K, "dtype": gw.dtype, "us_per_call": gq,
                                   "calls": 10000}
    torch.cuda.empty_cache()
    return out


def time_decode(mk, stream, loop, ncalls=10000, per_graph=100):
    """µs per call of the call mk(stream) made `ncalls` times back to back:
    from a Python loop, from a loop in C (if built), and captured
    `per_graph` to a HIP graph and replayed."""
    import torch
    call = mk(stream)
    for _ in range(200):
        run(call)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(ncalls):
        run(call)
    e1.record(stream)
    torch.cuda.synchronize()
    out = {"python_loop": round(e0.elapsed_time(e1) * 1e3 / ncalls, 3)}
    if loop is not None:
        out["c_loop"] = round(time_c_loop(loop, call, ncalls, stream), 3)
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    gcall = mk(cs)
    with torch.cuda.stream(cs):
        for _ in range(10):
            run(gcall)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for _ in range(per_graph):
            run(gcall)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(ncalls // per_graph):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    out["hip_graph"] = round(e0.elapsed_time(e1) * 1e3 / ncalls, 3)
    del g
    return out


def _host_cpu():
    """(usable cores, visible cores, CPU model) of this host."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, os.cpu_count() or usable, model


def cpu_baseline(min_seconds=10.0, sample_rows=1024):
    """The oracle (plain C, double) on a bounded sample of the headline
    workload: the first `sample_rows` rows of the bf16 residual 16384 x 4096
    step (residual forward, then the backward with dres), repeated until
    `min_seconds` have passed.  Once on one thread, then on all the cores
    this process may use: the sample's rows split into one slice per thread,
    each thread calling the oracle on its slice (ctypes releases the GIL for
    the call).  GB/s counts the step's algorithmic bytes for the rows done."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    from bwd_rmsnorm_fwd_amd import synth

    wl = synth.WORKLOADS[HEADLINE]
    R = sample_rows
    full_x = wl.x()
    x = synth.to_f64(full_x[:R], wl.dtype)
    del full_x
    res = synth.to_f64(wl.res()[:R], wl.dtype)
    dy = synth.to_f64(wl.dy()[:R], wl.dtype)
    dres = synth.to_f64(wl.dres()[:R], wl.dtype)
    w = synth.to_f64(wl.w(), wl.dtype)
    oracle.rmsnorm_fwd(x[:2], w, wl.eps)  # load / build outside the timing

    def one(lo, hi):
        h, _, r = oracle.rmsnorm_residual_fwd(x[lo:hi], res[lo:hi], w, wl.eps, oracle.H_BF16)
        oracle.rmsnorm_bwd(dy[lo:hi], h, w, wl.eps, rstd=r, dres=dres[lo:hi])

    def timed(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                return n, el

    step_bytes_per_row = (fwd_bytes(wl.rows, wl.H, 2, residual=True)
                          + bwd_bytes(wl.rows, wl.H, 2, dres=True)) / wl.rows
    n1, el1 = timed(lambda: one(0, R))
    usable, visible, model = _host_cpu()
    bounds = np.linspace(0, R, usable + 1).astype(int)
    with ThreadPoolExecutor(max_workers=usable) as ex:
        def all_cores():
            list(ex.map(lambda k: one(bounds[k], bounds[k + 1]), range(usable)))
        nn, eln = timed(all_cores)
    gbs1 = n1 * R * step_bytes_per_row / el1 / 1e9
    gbsn = nn * R * step_bytes_per_row / eln / 1e9
    full_ms = lambda gbs: (step_bytes_per_row * wl.rows) / (gbs * 1e9) * 1e3
    return {"value": round(gbsn, 4), "unit": "GB/s", "cores": usable, "kind": "oracle",
            "sample": f"rows 0-{R - 1} of the bf16 residual 16384x4096 step (residual forward + "
                      f"backward with dres, inputs widened to float64): {nn} passes in "
                      f"{eln:.1f} s on {usable} threads (one row slice each)",
            "ms_per_full_step": round(full_ms(gbsn), 1),
            "single_thread": {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                              "passes": n1, "seconds": round(el1, 1),
                              "ms_per_full_step": round(full_ms(gbs1), 1)},
            "host": {"usable_cores": usable, "visible_cpus": visible, "cpu_model": model,
                     "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}}


def load_traffic(kernel_name):
    """HBM traffic per launch of a kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(kernel_name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


# ---------------------------------------------------------------- suite

def time_calls(calls_per_set, k, reps, warmup, stream, burst=16):
    """Per-launch µs of each call group over rotating sets: `reps` bursts of
    `burst` back-to-back groups, events only at the burst ends.  Returns one
    list (µs per group, one entry per burst) for each prefix of the group:
    entry j times calls 0..j together, so a group (a, b) gives a alone and
    a followed by b."""
    import torch
    for i in range(warmup):
        for c in calls_per_set[i % k]:
            run(c)
    torch.cuda.synchronize()
    n = len(calls_per_set[0])
    out = []
    for j in range(n):
        res = []
        for r in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(burst):
                grp = calls_per_set[(r * burst + i) % k]
                for c in grp[: j + 1]:
                    run(c)
            e1.record(stream)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e3 / burst)
        out.append(res)
    return out


def summarise(name, us, nbytes, extra=None):
    med = statistics.median(us)
    p95 = sorted(us)[min(len(us) - 1, int(0.95 * len(us)))]
    gbs = nbytes / (med * 1e-6) / 1e9
    d = {"name": name, "us_median": round(med, 3), "us_p95": round(p95, 3),
         "us_mean": round(statistics.mean(us), 3), "bytes": nbytes, "GB_s": round(gbs, 1),
         "pct_peak": round(100 * gbs / PEAK_GBS, 2)}
    if extra:
        d.update(extra)
    return d


def wide_workloads():
    """Rows wider than every configured workload (bf16, 128 MB per tensor):
    the forward's 512 x 4 tile at 16384, the backward's register tile there,
    its row-in-LDS kernel at 32768 and its streaming kernel at 65536 and with
    a residual-stream gradient at 32768."""
    from bwd_rmsnorm_fwd_amd import synth
    wide = [synth.Workload(f"wide_bf16_{r}x{h}", synth.BF16, r, h, 1e-6, 701 + k, 711 + k, 721 + k,
                           731 + k, 741 + k)
            for k, (r, h) in enumerate(((4096, 16384), (2048, 32768), (1024, 65536)))]
    wide.append(synth.Workload("wide_bf16_residual_2048x32768", synth.BF16, 2048, 32768, 1e-6,
                               751, 752, 753, 754, 755, residual=True))
    return wide


def workload_by_name(name):
    from bwd_rmsnorm_fwd_amd import synth
    if name in synth.WORKLOADS:
        return synth.WORKLOADS[name]
    return {w.name: w for w in wide_workloads()}[name]


def suite(path, reps=30, warmup=20):
    import torch
    from bwd_rmsnorm_fwd_amd import synth

    stream = torch.cuda.current_stream()
    out = []

    def emit(d):
        out.append(d)
        print(json.dumps(d), file=sys.stderr, flush=True)

    wide = [w for w in wide_workloads() if not w.residual]
    plain = [synth.WORKLOADS[n] for n in ("c1_f32_64x896", "c2_bf16_4096x4096",
                                          "c5a_bf16_262144x128", "c5b_bf16_8192x8192")]
    for wl in plain + wide:
        name = wl.name
        is_wide = wl in wide
        sets = Sets(wl)
        C = Calls(sets, stream)
        e = sets.e
        meta = {"workload": name, "cold_sets": sets.k}
        (tf,) = time_calls([(C.fwd(s),) for s in sets.sets], sets.k, reps, warmup, stream)
        tr, tb = time_calls([(C.bwd_rows(s), C.dw_reduce(s)) for s in sets.sets], sets.k, reps,
                            warmup, stream)
        (td,) = time_calls([(C.dw_reduce(s),) for s in sets.sets], sets.k, reps, warmup, stream)
        (ts, ) = time_calls(step_plan(C, sets), sets.k, reps, max(warmup, sets.k), stream)[2:]
        emit(summarise(f"{name}/fwd", tf, fwd_bytes(wl.rows, wl.H, e), meta))
        emit(summarise(f"{name}/bwd_rows", tr, bwd_rows_bytes(wl.rows, wl.H, e), meta))
        emit(summarise(f"{name}/dw_reduce", td, wl.H * e, meta))
        emit(summarise(f"{name}/bwd", tb, bwd_bytes(wl.rows, wl.H, e), meta))
        emit(summarise(f"{name}/step_fwd_bwd", ts,
                       fwd_bytes(wl.rows, wl.H, e) + bwd_bytes(wl.rows, wl.H, e), meta))
        if is_wide:
            del sets, C
            torch.cuda.empty_cache()
            continue
        # Backward that recomputes r from x instead of reading the saved rstd
        # (4 bytes per row fewer; one more row reduction).
        (tq,) = time_calls([(C.bwd_rows(s, saved_rstd=False),) for s in sets.sets], sets.k, reps,
                           warmup, stream)
        emit(summarise(f"{name}/bwd_rows_recompute_rstd", tq,
                       bwd_rows_bytes(wl.rows, wl.H, e) - 4 * wl.rows, meta))
        # Warm-cache forward (same buffers every call): labelled, not HBM.
        (wf,) = time_calls([(C.fwd(sets.sets[0]),)], 1, reps, warmup, stream)
        emit(summarise(f"{name}/fwd_warm_cache", wf, fwd_bytes(wl.rows, wl.H, e),
                       {"workload": name, "note": "same buffers each call; not HBM-bound"}))
        del sets, C
        torch.cuda.empty_cache()

    wide_res = workload_by_name("wide_bf16_residual_2048x32768")
    for wl in (synth.WORKLOADS["c4_bf16_residual_16384x4096"], wide_res):
        sets = Sets(wl, residual=True, dres=True)
        C = Calls(sets, stream)
        meta = {"workload": wl.name, "cold_sets": sets.k}
        (tf,) = time_calls([(C.residual_fwd(s),) for s in sets.sets], sets.k, reps, warmup, stream)
        tr, tb = time_calls([(C.bwd_rows(s, x_key="h", dres=True), C.dw_reduce(s))
                             for s in sets.sets], sets.k, reps, warmup, stream)
        emit(summarise(f"{wl.name}/residual_fwd", tf, fwd_bytes(wl.rows, wl.H, 2, residual=True),
                       meta))
        emit(summarise(f"{wl.name}/bwd_rows_dres", tr,
                       bwd_rows_bytes(wl.rows, wl.H, 2, dres=True), meta))
        emit(summarise(f"{wl.name}/bwd_dres", tb, bwd_bytes(wl.rows, wl.H, 2, dres=True), meta))
        del sets, C
        torch.cuda.empty_cache()

    # Decode: 10k back-to-back calls on one stream, µs per call: from a
    # Python loop, from a loop in C, and replayed from a HIP graph.
    CL = c_loops()
    wl = synth.WORKLOADS["c3_bf16_decode_1x896"]
    sets = Sets(wl, k=1)
    C = Calls(sets, stream)
    s = sets.sets[0]
    ncalls = 10000
    for splits in (0, 1, 4, 8, 16):
        if splits == 0:
            call = C.fwd(s)
            label = "row_kernel"
        else:
            partials = torch.empty(splits, dtype=torch.float32, device="cuda")
            call = C.splitrow(s, partials, splits)
            label = f"splitrow_S{splits}"
        for _ in range(200):
            run(call)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(ncalls):
            run(call)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / ncalls
        emit({"name": f"{wl.name}/{label}", "us_per_call": round(us, 3), "calls": ncalls,
              "launches_per_call": 1 if splits == 0 else 2,
              "bytes": fwd_bytes(1, wl.H, 2), "workload": wl.name})
        if CL is not None:
            loop = CL.bench_fwd_loop if splits == 0 else CL.bench_splitrow_loop
            uc = time_c_loop(loop, call, ncalls, stream)
            emit({"name": f"{wl.name}/{label}_c_loop", "us_per_call": round(uc, 3),
                  "calls": ncalls, "launches_per_call": 1 if splits == 0 else 2,
                  "bytes": fwd_bytes(1, wl.H, 2), "workload": wl.name,
                  "note": "calls made by a loop in C (no Python per call)"})
        # The same calls captured once in a HIP graph (100 per graph) and
        # replayed: the host launch cost per call disappears.
        per_graph, replays = 100, ncalls // 100
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        Cg = Calls(sets, cs)
        gcall = Cg.fwd(s) if splits == 0 else Cg.splitrow(s, partials, splits)
        with torch.cuda.stream(cs):
            for _ in range(10):
                run(gcall)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            for _ in range(per_graph):
                run(gcall)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ug = e0.elapsed_time(e1) * 1e3 / (per_graph * replays)
        emit({"name": f"{wl.name}/{label}_hip_graph", "us_per_call": round(ug, 3),
              "calls": per_graph * replays, "calls_per_graph": per_graph,
              "launches_per_call": 1 if splits == 0 else 2,
              "bytes": fwd_bytes(1, wl.H, 2), "workload": wl.name})
        del g
    del sets, C
    torch.cuda.empty_cache()

    # Split-K decode projection (q_proj 896 -> 1024): 10k calls per split
    # count, plain and captured in a HIP graph.
    import numpy as np
    from bwd_rmsnorm_fwd_amd import binding as B
    gw = synth.GEMV_WORKLOADS["q_proj_bf16_1024x896"]
    A = torch.from_numpy(gw.A().view(np.int16)).view(torch.bfloat16).cuda()
    xv = torch.from_numpy(gw.x().view(np.int16)).view(torch.bfloat16).cuda()
    yv = torch.empty(gw.N, dtype=torch.bfloat16, device="cuda")
    L = B.lib()
    gbytes = (gw.N * gw.K + gw.K + gw.N) * 2
    for splits in gw.splits:
        parts = torch.empty(max(B.decode_gemv_partials_count(gw.N, splits), 1), device="cuda")

        def gcall(st):
            return (L.decode_gemv_splitk,
                    (ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(xv.data_ptr()),
                     ctypes.c_void_p(yv.data_ptr()), ctypes.c_void_p(parts.data_ptr()),
                     parts.numel(), gw.N, gw.K, splits, B.BF16, ctypes.c_void_p(st.cuda_stream)))
        call = gcall(stream)
        for _ in range(200):
            run(call)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(ncalls):
            run(call)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / ncalls
        emit({"name": f"{gw.name}/gemv_S{splits}", "us_per_call": round(us, 3), "calls": ncalls,
              "launches_per_call": 1 if splits == 1 else 2, "bytes": gbytes,
              "GB_s": round(gbytes / us / 1e3, 1), "workload": gw.name})
        if CL is not None:
            uc = time_c_loop(CL.bench_gemv_loop, call, ncalls, stream)
            emit({"name": f"{gw.name}/gemv_S{splits}_c_loop", "us_per_call": round(uc, 3),
                  "calls": ncalls, "launches_per_call": 1 if splits == 1 else 2, "bytes": gbytes,
                  "GB_s": round(gbytes / uc / 1e3, 1), "workload": gw.name,
                  "note": "calls made by a loop in C (no Python per call)"})
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        c2 = gcall(cs)
        with torch.cuda.stream(cs):
            for _ in range(10):
                run(c2)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            for _ in range(100):
                run(c2)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(ncalls // 100):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ug = e0.elapsed_time(e1) * 1e3 / ncalls
        emit({"name": f"{gw.name}/gemv_S{splits}_hip_graph", "us_per_call": round(ug, 3),
              "calls": ncalls, "launches_per_call": 1 if splits == 1 else 2, "bytes": gbytes,
              "GB_s": round(gbytes / ug / 1e3, 1), "workload": gw.name})
        del g
    with open(path, "w") as f:
        for d in out:
            f.write(json.dumps(d) + "\n")


# ---------------------------------------------------------------- counter passes

COUNTER_WORKLOADS = ["c1_f32_64x896", "c2_bf16_4096x4096", "c5a_bf16_262144x128",
                     "c5b_bf16_8192x8192", "c4_bf16_residual_16384x4096",
                     "wide_bf16_2048x32768", "wide_bf16_1024x65536",
                     "wide_bf16_residual_2048x32768", "c3_bf16_decode_1x896",
                     "q_proj_bf16_1024x896"]


def counters_pass(n, plan_out=None):
    """Every workload's kernels, n launches each on rotating buffer sets, with
    no timing: the program that rocprofv3 trace and counter passes run over.
    Per workload, in COUNTER_WORKLOADS order: n forwards back to back, then n
    times the backward row pass followed by its dw reduce (residual forward
    and the row pass with dres for the residual workload) -- the bursts the
    per-kernel timings of this file measure; decode runs n one-row forwards,
    then n split-row forwards for each of 1, 4, 8 and 16 splits; the decode
    projection n calls per split count.  plan_out, if given, receives the
    launch plan as JSON: per workload, the kernels (named by the library's dry
    run) in launch order, so that a trace can be cut into workloads."""
    import torch

    stream = torch.cuda.current_stream()
    plan = []
    for name in COUNTER_WORKLOADS:
        if name.startswith("q_proj"):
            plan += gemv_pass(name, n, stream)
            continue
        wl = workload_by_name(name)
        residual = wl.residual
        sets = Sets(wl, k=1 if wl.rows == 1 else None, residual=residual, dres=residual)
        C = Calls(sets, stream)
        if wl.rows == 1:
            groups = [("fwd", [C.fwd(s) for s in sets.sets])]
            for S in (1, 4, 8, 16):
                parts = torch.empty(S, dtype=torch.float32, device="cuda")
                groups.append((f"splitrow_S{S}", [C.splitrow(s, parts, S) for s in sets.sets]))
            for label, calls in groups:
                for i in range(n):
                    run(calls[i % len(calls)])
                plan.append({"workload": name, "op": label, "repeats": n,
                             "kernels": [k for ks in kernel_names(C, calls[:1]) for k in ks]})
        else:
            seq = step_plan(C, sets, residual=residual)
            meta = {"rows": wl.rows, "H": wl.H, "dtype": wl.dtype, "residual": residual,
                    "cold_sets": sets.k}
            for label, idx in (("fwd", (0,)), ("bwd_rows+dw_reduce", (1, 2))):
                for i in range(n):
                    for j in idx:
                        run(seq[i % sets.k][j])
                plan.append(dict(meta, workload=name, op=label, repeats=n,
                                 kernels=[k for ks in kernel_names(C, [seq[0][j] for j in idx])
                                          for k in ks]))
        torch.cuda.synchronize()
        del sets, C
        torch.cuda.empty_cache()
    if plan_out:
        with open(plan_out, "w") as f:
            json.dump(plan, f, indent=1)


def gemv_pass(name, n, stream):
    """The split-K decode projection, n calls for each split count; returns
    its part of the launch plan."""
    import numpy as np
    import torch
    from bwd_rmsnorm_fwd_amd import binding as B
    from bwd_rmsnorm_fwd_amd import synth
    gw = synth.GEMV_WORKLOADS[name]
    A = torch.from_numpy(gw.A().view(np.int16)).view(torch.bfloat16).cuda()
    xv = torch.from_numpy(gw.x().view(np.int16)).view(torch.bfloat16).cuda()
    yv = torch.empty(gw.N, dtype=torch.bfloat16, device="cuda")
    L = B.lib()
    plan = []
    for splits in gw.splits:
        parts = torch.empty(max(B.decode_gemv_partials_count(gw.N, splits), 1), device="cuda")
        call = (L.decode_gemv_splitk,
                (ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(xv.data_ptr()),
                 ctypes.c_void_p(yv.data_ptr()), ctypes.c_void_p(parts.data_ptr()), parts.numel(),
                 gw.N, gw.K, splits, B.BF16, ctypes.c_void_p(stream.cuda_stream)))
        for _ in range(n):
            run(call)
        plan.append({"workload": name, "op": f"gemv_S{splits}", "repeats": n,
                     "kernels": [l.split(" grid=")[0] for l in B.launches_of(call[0], *call[1])]})
    torch.cuda.synchronize()
    return plan


# ---------------------------------------------------------------- entry

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU needs some milliseconds of load before its clocks settle; the
    # per-configuration table and the per-kernel bursts run first, so even a
    # short warm-up starts from a busy GPU.
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--suite", default=None, help="also measure every workload into this file")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration table (headline step only)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-ref-mb", type=int, default=0,
                    help="after the step, run a plain device copy of this many MiB (reference "
                         "kernel of known size for scaling rocprofv3 byte counters)")
    ap.add_argument("--counters-pass", type=int, default=0, metavar="N",
                    help="instead of timing, launch every workload's kernels N times each "
                         "(the program for rocprofv3 counter passes), then the --copy-ref-mb copy")
    ap.add_argument("--plan-out", default=None,
                    help="with --counters-pass: write the launch plan (JSON) to this file")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the RMSNorm library runs on a single MI355X (rows "
              "would shard across GPUs with no exchange except one dw all-reduce, which this "
              "library does not provide); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()
    if args.counters_pass:
        counters_pass(args.counters_pass, args.plan_out)
        copy_ref(args.copy_ref_mb)
        print(json.dumps({"counters_pass": args.counters_pass, "workloads": COUNTER_WORKLOADS,
                          "copy_ref_bytes": args.copy_ref_mb << 20}), flush=True)
        return
    # Every configuration first (this also brings the GPU to its working
    # clocks), then the headline step: W warm-up steps and K timed steps.
    configs = config_table() if not args.no_configs else None
    r = bench_step(args.steps, args.warmup)
    wl = r["wl"]
    total_bytes = r["fwd_bytes"] + r["bwd_bytes"]
    value = total_bytes / (r["ms_step"] * 1e-3) / 1e9
    # The dominant kernel: the longer of the residual forward and the
    # backward row pass.  The forward is timed in a burst of itself.  The row
    # pass is timed in a burst of itself and in a burst of (row pass, dw
    # reduce) pairs, the way rmsnorm_bwd runs it; both figures bound the
    # kernel from above (the pair's includes the reduce), and the smaller one
    # is used: on some parts the row pass runs 5-12% slower back to back with
    # itself than between reduces or inside the steps, where traces put it
    # within 1% of the forward.  (Events around each launch would add their
    # own 5-6 µs per launch, by the trace of the same run.)
    dom_name, dom_us, dom_bytes, basis, rows_us = pick_roofline(r)
    ach = dom_bytes / (dom_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused residual-add + RMSNorm fwd+bwd bf16 rows=16384 (B=4,T=4096) "
                               "H=4096 eps=1e-6 (x,res~N(0,1), w~U(0.5,1.5), dy,dres~N(0,1e-2)); "
                               "bwd adds dres into dh",
                   "rows": wl.rows, "H": wl.H, "cold_cache_buffer_sets": r["k"],
                   "bytes_per_step": total_bytes},
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "fwd_us": round(r["fwd_us"], 3),
        "bwd_us": round(r["bwd_us"], 3),
        "bwd_rows_us": round(r["rows_us"], 3),
        "fwd_pct_peak": _pct(r["fwd_bytes"], r["fwd_us"])[1],
        "bwd_pct_peak": _pct(r["bwd_bytes"], r["bwd_us"])[1],
        "event_span_ms_per_step": round(r["span_ms"], 5),
        "kernels": [k for ks in r["names"] for k in ks],
        "timing": f"value/ms_per_step: wall clock over the timed steps (no per-kernel events); "
                  f"per-kernel µs: HIP events around a burst of {r['burst']} back-to-back "
                  f"launches (fwd alone, bwd row pass alone, row pass + dw reduce), run before "
                  f"the warm-up steps",
        "roofline": {
            "kernel": dom_name,
            "bound": "hbm",
            "achieved": round(ach, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach / PEAK_GBS, 4),
            "traffic": load_traffic(dom_name),
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_us, 3),
            "timed_as": basis,
        },
    }
    e = 4 if wl.dtype == "f32" else 2
    ceil = ceilings_of(wl, e, wl.residual, _pct(r["fwd_bytes"], r["fwd_us"])[0],
                       _pct(r["rows_bytes"], rows_us)[0], torch.cuda.current_stream())
    line.update(ceil)
    if configs is not None:
        line["configs"] = configs
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    if args.suite:
        suite(args.suite)
    if args.copy_ref_mb:
        copy_ref(args.copy_ref_mb)
        line["copy_ref_bytes"] = args.copy_ref_mb << 20
    print(json.dumps(line), flush=True)


def copy_ref(mb):
    """A plain device copy of `mb` MiB, three times: a kernel of known size
    whose counters scale the byte counters of the others."""
    if not mb:
        return
    import torch
    src = torch.ones(mb << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
