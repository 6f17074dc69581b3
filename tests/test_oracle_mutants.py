"""The oracle pins have teeth: each planted mistake in a copy of the oracle's C
source (compiled here, on the CPU) must make the pin suite fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "trimul_oracle.c")

MUTANTS = {
    "unbiased_variance": ("var /= (double)L;", "var /= (double)(L - 1);"),
    "eps_outside_sqrt": ("1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    "dropped_beta": ("* (double)gamma[d] + (double)beta[d]", "* (double)gamma[d]"),
    "sigmoid_sign": ("1.0 / (1.0 + exp(-t))", "1.0 / (1.0 + exp(t))"),
    "a_gated_by_b_gate": ("double ga = dot_row(w->g_in + (size_t)c * D, x, D);",
                          "double ga = dot_row(w->g_in + (size_t)(C + c) * D, x, D);"),
    "b_unmasked": ("b[c] = m * pb * sigm(gb)", "b[c] = pb * sigm(gb)"),
    "incoming_as_outgoing": ("ta = a + ((size_t)k * N + i) * C;", "ta = a + ((size_t)i * N + k) * C;"),
    "outgoing_transposed_b": ("tb = b + ((size_t)j * N + k) * C;", "tb = b + ((size_t)k * N + j) * C;"),
    "last_k_dropped": ("for (int k = 0; k < N; ++k) {\n                    const double *ta, *tb;",
                       "for (int k = 0; k < N - 1; ++k) {\n                    const double *ta, *tb;"),
    "gate_row_stride": ("dot_row(w->g_out + (size_t)d * D, x, D)", "dot_row(w->g_out + (size_t)d, x, D)"),
    "ln_out_over_wrong_params": ("layer_norm(o, C, w->ln_out_w, w->ln_out_b", "layer_norm(o, C, w->ln_in_w, w->ln_out_b"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib),
                    str(msrc), "-lm"], check=True)
    env = dict(os.environ, TRIMUL_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])


# The hand-worked examples (tests/golden) alone, without any test that recomposes
# the formula from library routines, catch every planted mistake a no-mask
# example can see (b_unmasked needs a mask; the other pins catch it).
VALUE_PINNED = sorted(set(MUTANTS) - {"b_unmasked"})


@pytest.mark.parametrize("name", VALUE_PINNED)
def test_hand_worked_values_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib),
                    str(msrc), "-lm"], check=True)
    env = dict(os.environ, TRIMUL_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-k", "hand_worked", os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "hand-worked values did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
