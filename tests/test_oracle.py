"""CPU tests of the oracle: every pin must hold, and deliberately broken builds of the oracle
(a dropped term, a wrong sign, a wrong index, a transposed operand, a wrong order) must each
fail at least one pin. The broken builds are made here, on the CPU, from a patched copy of
oracle.c; the real oracle.c is never modified."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=True)
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# (description, text in oracle.c, replacement)
MUTANTS = [
    ("gemm drops the last k term", "for (int64_t k = 0; k < K; ++k) {\n      const double a",
     "for (int64_t k = 0; k < K - 1; ++k) {\n      const double a"),
    ("gemm transposes B", "const double* b = B + k * N;\n      for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];",
     "for (int64_t j = 0; j < N; ++j) c[j] += a * B[(j % K) * N + (k % N)];"),
    ("gemm transposes A", "const double a = A[i * K + k];", "const double a = A[(k % M) * K + (i % K)];"),
    ("bf16 decode shifted", "((uint32_t)h) << 16", "((uint32_t)h) << 15"),
    ("AG ring runs the other way", "out[t] = ((r - t) % P + P) % P;", "out[t] = (r + t) % P;"),
    ("RS own chunk first", "for (int i = 0; i < P - 1; ++i) out[i] = (r + 1 + i) % P;\n  out[P - 1] = r;",
     "for (int i = 0; i < P; ++i) out[i] = (r + i) % P;"),
    ("RS drops one incoming partial", "for (int i = 1; i < P; ++i) {\n        const int q = ((r - i) % P + P) % P;\n        const float* pq",
     "for (int i = 2; i < P; ++i) {\n        const int q = ((r - i) % P + P) % P;\n        const float* pq"),
    ("RS subtracts partials", "out[e] += (double)pq[e];", "out[e] -= (double)pq[e];"),
    ("RS adds its own slot instead of a peer", "const int q = ((r - i) % P + P) % P;\n        const float* pq",
     "const int q = ((r - i + 1) % P + P) % P;\n        const float* pq"),
    ("AG writes by position, not slice", "gemm_f64(xs, w, Y + (int64_t)s * m * N, m, K, N);",
     "gemm_f64(xs, w, Y + (int64_t)t * m * N, m, K, N);"),
    ("sampled RS forgets partials", "v += (double)partials[q][rows[t] * N + cols[t]];", "(void)q;"),
    ("sampled AG reads the wrong slice", "const int64_t s = rows[t] / m;", "const int64_t s = (rows[t] / m + 1) % P;"),
]


def _run_pins_in_child(lib):
    return subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib],
                          capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, OMP_NUM_THREADS="2"))


def test_pin_runner_passes_on_real_oracle(tmp_path):
    """Control for the mutation check: the unmodified oracle, run the same way, passes."""
    lib = oracle.build(force=True, out=str(tmp_path / "libcontrol.so"))
    res = _run_pins_in_child(lib)
    assert res.returncode == 0 and "all pins hold" in res.stdout, res.stdout + res.stderr


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, desc, old, new):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor for '{desc}' not found in oracle.c"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(mutant_c), out=lib)
    # run in a child: a broken build may also crash (killed by a signal), which counts as caught
    res = _run_pins_in_child(lib)
    caught = (res.returncode == 1 and "PIN FAILED" in res.stdout) or res.returncode < 0
    assert caught, f"no pin caught: {desc}\n{res.stdout}{res.stderr}"
