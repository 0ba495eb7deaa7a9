"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible slip in a copy of oracle/rmsnorm_oracle.c
(a dropped term, a wrong sign, power or index, a transposed operand, a wrong
rounding), builds it, and runs tests/test_oracle_pins.py against that build in
a subprocess (RMSNORM_ORACLE_LIB): at least one pin must fail.  The unmutated
source, built the same way, must pass every pin, so a broken harness cannot
make the mutants look caught.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rmsnorm_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in the oracle source, replacement); each text occurs once.
MUTANTS = [
    ("eps dropped", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
    ("sum instead of mean", "sqrt(ss / (double)H + eps)", "sqrt(ss + eps)"),
    ("sqrt missing", "1.0 / sqrt(ss / (double)H + eps)", "1.0 / (ss / (double)H + eps)"),
    ("r not inverted", "1.0 / sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H + eps)"),
    ("forward without w", "y[i * H + j] = w[j] * xr[j] * r;", "y[i * H + j] = xr[j] * r;"),
    ("forward w index shifted", "y[i * H + j] = w[j] * xr[j] * r;",
     "y[i * H + j] = w[(j + 1) % H] * xr[j] * r;"),
    ("residual subtracts", "double s = x[k] + res[k];", "double s = x[k] - res[k];"),
    ("residual rounded to fp32 for bf16",
     "else if (h_kind == ORACLE_H_BF16) s = oracle_round_bf16(s);",
     "else if (h_kind == ORACLE_H_BF16) s = oracle_round_f32(s);"),
    ("c without 1/H", "        c /= (double)H;\n", ""),
    ("dx sign", "r * (w[j] * dyr[j] - xr[j] * r * r * c)", "r * (w[j] * dyr[j] + xr[j] * r * r * c)"),
    ("dx r instead of r^2", "xr[j] * r * r * c", "xr[j] * r * c"),
    ("dw without r", "dw[j] += dyr[j] * xr[j] * r;", "dw[j] += dyr[j] * xr[j];"),
    ("dw with w", "dw[j] += dyr[j] * xr[j] * r;", "dw[j] += w[j] * dyr[j] * xr[j] * r;"),
    ("dres ignored", "if (dres) g += dres[i * H + j];", ""),
    ("saved rstd ignored", "double r = rstd ? rstd[i] : row_rstd(xr, H, eps);",
     "double r = row_rstd(xr, H, eps);"),
    ("c without w", "c += w[j] * dyr[j] * xr[j];", "c += dyr[j] * xr[j];"),
    ("bf16 keeps 7 bits", "int q = e - 8;", "int q = e - 7;"),
    ("bf16 truncates", "nearbyint(ldexp(v, -q))", "trunc(ldexp(v, -q))"),
    ("gemv transposed", "s += A[n * K + k] * x[k];", "s += A[k * N + n] * x[k];"),
    ("dw not cleared", "for (int64_t j = 0; j < H; ++j) dw[j] = 0.0;",
     "for (int64_t j = 0; j < H; ++j) dw[j] = 1.0;"),
]


def _run_pins(lib_path):
    env = dict(os.environ, RMSNORM_ORACLE_LIB=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _build(tmp, name, text):
    src = os.path.join(tmp, f"{name}.c")
    with open(src, "w") as f:
        f.write(text)
    return oracle.build(src, os.path.join(tmp, f"{name}.so"))


def test_every_mutant_fails_a_pin(tmp_path):
    base = open(SRC).read()
    tmp = str(tmp_path)
    jobs = [("unmutated", base)]
    for i, (name, old, new) in enumerate(MUTANTS):
        assert base.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
        jobs.append((f"m{i:02d}", base.replace(old, new)))
    libs = [(name, _build(tmp, name, text)) for name, text in jobs]
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda nl: _run_pins(nl[1]), libs))
    rc0, out0 = results[0]
    assert rc0 == 0, "the unmutated oracle must pass every pin:\n" + out0
    survivors = [MUTANTS[i][0] for i, (rc, _) in enumerate(results[1:]) if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
