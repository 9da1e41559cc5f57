"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/oracle.c with one plausible slip (a swapped
nibble, a wrong offset, a dropped term, a transposed operand ...), compiled
on the CPU into a temporary library. The pin suite (test_oracle_pins.py) is
run against it in a subprocess and must fail.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "int4_nibbles_swapped": ("(i % 2 == 0) ? (byte & 0xF) : ((byte >> 4) & 0xF)",
                             "(i % 2 == 1) ? (byte & 0xF) : ((byte >> 4) & 0xF)"),
    "int4_offset_7": ("return (double)(nib - 8);", "return (double)(nib - 7);"),
    "int2_bits_reversed": ("(byte >> (2 * (int)(i % 4))) & 0x3", "(byte >> (2 * (int)(3 - i % 4))) & 0x3"),
    "int2_offset_1": ("return (double)(code - 2);", "return (double)(code - 1);"),
    "int8_unsigned": ("if (v >= 128)\n            v -= 256;", ""),
    "scale_dropped": ("y[s * O + o] = (float)(acc * scale);", "y[s * O + o] = (float)acc;"),
    "last_column_dropped": ("for (long i = 0; i < I; ++i) {", "for (long i = 0; i + 1 < I; ++i) {"),
    "x_column_major": ("const float *xs = x + s * I;", "const float *xs = x + s * (I > 1 ? 1 : 0);"),
    "y_transposed": ("y[s * O + o] = (float)(acc * scale);", "y[o * S + s] = (float)(acc * scale);"),
    "null_scale_zero": ("double scale = scales ? (double)scales[o] : 1.0;",
                        "double scale = scales ? (double)scales[o] : 0.0;"),
    "f32_byte_offset": ("memcpy(&f, row + 4 * i, sizeof f);", "memcpy(&f, row + 2 * i, sizeof f);"),
    "sign_flipped": ("acc += t;", "acc -= t;"),
    "sum_in_float": ("double acc = 0.0, mag = 0.0;", "float acc = 0.0f; double mag = 0.0;"),
    # bound magnitude A (every parity tolerance is 1e-5 * A + 1e-30)
    "bound_times_100": ("absb[s * O + o] = mag * fabs(scale);", "absb[s * O + o] = 100.0 * mag * fabs(scale);"),
    "bound_signed_sum": ("mag += fabs(t);", "mag += t;"),
    "bound_scale_dropped": ("absb[s * O + o] = mag * fabs(scale);", "absb[s * O + o] = mag;"),
    "gs_bound_times_100": ("absb[s * O + o] = magnitude;", "absb[s * O + o] = 100.0 * magnitude;"),
    "gs_bound_signed_sum": ("group_mag += fabs(prod);", "group_mag += prod;"),
    # group-wise scales
    "gs_group_shifted": ("long first = g * gs, end", "long first = g * gs + 1, end"),
    "gs_scales_transposed": ("const float *srow = scales + o * ng;", "const float *srow = scales + o;"),
    "gs_scale_dropped": ("total += gscale * group_sum;", "total += group_sum;"),
    "gs_last_group_dropped": ("for (long g = 0; g < ng; ++g) {", "for (long g = 0; g + 1 < ng; ++g) {"),
    "gs_group_scale_of_next": ("double gscale = (double)srow[g];", "double gscale = (double)srow[(g + 1) % ng];"),
    # SiLU-gated product
    "silu_exp_sign": ("double silu = z / (1.0 + exp(-z));", "double silu = z / (1.0 + exp(z));"),
    "silu_gate_dropped": ("double silu = z / (1.0 + exp(-z));", "double silu = z;"),
}


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert old in src, "mutation anchor for %s not found" % name
    msrc = src.replace(old, new, 1)
    cpath = os.path.join(tmp, name + ".c")
    lpath = os.path.join(tmp, name + ".so")
    with open(cpath, "w") as f:
        f.write(msrc)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
                    cpath, "-o", lpath, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_UNDER_TEST=lpath, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_gs_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_ffn_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


@pytest.mark.slow
def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run_mutant, n, o, w, tmp) for n, (o, w) in MUTANTS.items()]
            results = [f.result() for f in futs]
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by the pins: %s" % survivors
    # a non-zero exit must come from failing tests, not a crash of the harness
    for n, rc, out in results:
        assert rc == 1, (n, rc, out)


def test_unmutated_source_passes_pins():
    """Control: the anchors exist and the real oracle passes (run in-process elsewhere)."""
    src = open(SRC).read()
    for name, (old, _) in MUTANTS.items():
        assert old in src, name
