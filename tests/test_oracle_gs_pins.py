"""Pins for the oracle's group-wise scale variant (one scale per row and
group of gs consecutive columns; the group-size field of the Vulkan tensor
description, colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 三).

- hand-worked matmuls (tests/golden/group_scale_examples.txt);
- exact rational brute force on tiny shapes, ragged last groups included;
- reductions: one group per row equals the per-row oracle bit for bit;
  equal scales in every group agree with it to an ulp;
- one-hot activations select scales[o, i // gs] * q[o, i] exactly;
- a zero group scale equals zeroing that group's activations, bit for bit;
- powers of two on all scales scale y exactly.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import brute
import golden_io
import oracle
import synth

F32, I8, I4, I2 = 0, 1, 2, 3
QUANT = (I8, I4, I2)


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)
    return np.abs(a - b) / sp


def gscales(g, O, I, gs, lo=0.001, hi=0.05):
    return g.uniform(lo, hi, size=(O, oracle.n_groups(I, gs))).astype(np.float32)


@pytest.mark.parametrize("case", golden_io.group_scale_examples(), ids=lambda c: c["name"])
def test_group_scale_worked_examples(case):
    y, a = oracle.matmul_gs(case["fmt"], case["w"], case["gscales"], case["gs"], case["x"], I=case["I"])
    np.testing.assert_array_equal(y, case["y"])
    np.testing.assert_array_equal(a, case["A"])  # hand-worked bound magnitudes (exact)
    yb = brute.matmul_gs_rounded(case["fmt"], case["w"], case["gscales"], case["gs"], case["x"], case["I"])
    np.testing.assert_array_equal(yb, case["y"])
    ab = brute.bound_gs_exact(case["fmt"], case["w"], case["gscales"], case["gs"], case["x"], case["I"])
    np.testing.assert_array_equal(np.array([[float(v) for v in r] for r in ab]), case["A"])


@pytest.mark.parametrize("fmt", QUANT + (F32,))
@pytest.mark.parametrize("shape,gs", [((3, 7, 1), 4), ((4, 16, 2), 8), ((2, 33, 3), 16), ((5, 64, 1), 64),
                                      ((2, 40, 2), 1)])
def test_group_scale_brute_force(fmt, shape, gs):
    O, I, S = shape
    g = synth.rng(3000 + 10 * fmt + O + gs)
    w = synth.weights(g, fmt, O, I)
    sc = gscales(g, O, I, gs)
    x = synth.activations(g, S, I)
    y, a = oracle.matmul_gs(fmt, w, sc, gs, x)
    yb = brute.matmul_gs_rounded(fmt, w, sc, gs, x, I)
    d = ulp_diff(y, yb)
    assert d.max() <= 1.0, d.max()
    assert np.mean(d == 0) >= 0.8
    # the bound magnitude against exact rationals (n exact terms summed in double)
    ab = brute.bound_gs_exact(fmt, w, sc, gs, x, I)
    for s_ in range(S):
        for o in range(O):
            v = ab[s_][o]
            err = abs(Fraction(float(a[s_, o])) - v)
            assert (err == 0) if v == 0 else float(err / v) <= 1e-12, (s_, o)


@pytest.mark.parametrize("fmt", QUANT)
@pytest.mark.parametrize("gs_over", [0, 5])
def test_single_group_equals_per_row_oracle(fmt, gs_over):
    O, I, S = 9, 300, 3
    g = synth.rng(3100 + fmt)
    w = synth.weights(g, fmt, O, I)
    sc = synth.scales(g, O, 0.001, 0.05)
    x = synth.activations(g, S, I)
    y_row, a_row = oracle.matmul(fmt, w, sc, x)
    y_gs, a_gs = oracle.matmul_gs(fmt, w, sc[:, None], I + gs_over, x)
    np.testing.assert_array_equal(y_gs, y_row)
    np.testing.assert_allclose(a_gs, a_row, rtol=1e-12)


@pytest.mark.parametrize("fmt", QUANT)
def test_equal_group_scales_match_per_row_oracle(fmt):
    O, I, S, gs = 12, 1000, 2, 64
    g = synth.rng(3200 + fmt)
    w = synth.weights(g, fmt, O, I)
    sc = synth.scales(g, O, 0.001, 0.05)
    x = synth.activations(g, S, I)
    y_row, _ = oracle.matmul(fmt, w, sc, x)
    y_gs, _ = oracle.matmul_gs(fmt, w, np.repeat(sc[:, None], oracle.n_groups(I, gs), axis=1), gs, x)
    assert ulp_diff(y_gs, y_row).max() <= 1.0


@pytest.mark.parametrize("fmt,I", [(I8, 256), (I4, 512), (I2, 1024)])
def test_one_hot_selects_group_scaled_code(fmt, I):
    gs = 64
    row = np.arange(256, dtype=np.uint8)[None, :]
    w = np.repeat(row, 2, axis=0)
    g = synth.rng(3300 + fmt)
    sc = gscales(g, 2, I, gs, 0.01, 3.0)
    q = np.array([float(v) for v in brute.codes(fmt, row[0].tobytes(), I)])
    cols = list(range(0, I, 7)) + [I - 1]
    x = np.zeros((len(cols), I), dtype=np.float32)
    x[np.arange(len(cols)), cols] = 1.0
    y, _ = oracle.matmul_gs(fmt, w, sc, gs, x)
    for s, c in enumerate(cols):
        for o in range(2):
            assert y[s, o] == np.float32(np.float64(sc[o, c // gs]) * q[c]), (s, c, o)


@pytest.mark.parametrize("fmt", QUANT)
def test_zero_group_scale_equals_zeroed_activations(fmt):
    O, I, S, gs = 6, 777, 3, 128
    g = synth.rng(3400 + fmt)
    w = synth.weights(g, fmt, O, I)
    sc = gscales(g, O, I, gs)
    x = synth.activations(g, S, I)
    for grp in (0, 3, oracle.n_groups(I, gs) - 1):  # first, middle, ragged last group
        sc0 = sc.copy()
        sc0[:, grp] = 0.0
        x0 = x.copy()
        x0[:, grp * gs:(grp + 1) * gs] = 0.0
        y_a, _ = oracle.matmul_gs(fmt, w, sc0, gs, x)
        y_b, _ = oracle.matmul_gs(fmt, w, sc, gs, x0)
        np.testing.assert_array_equal(y_a, y_b)


@pytest.mark.parametrize("fmt", QUANT)
def test_power_of_two_scales_scale_output_exactly(fmt):
    O, I, S, gs = 5, 500, 2, 64
    g = synth.rng(3500 + fmt)
    w = synth.weights(g, fmt, O, I)
    sc = gscales(g, O, I, gs)
    x = synth.activations(g, S, I)
    y, _ = oracle.matmul_gs(fmt, w, sc, gs, x)
    y8, _ = oracle.matmul_gs(fmt, w, sc * np.float32(8.0), gs, x)
    np.testing.assert_array_equal(y8, y * np.float32(8.0))


def test_group_scale_rejects_bad_arguments():
    w = np.zeros((2, 4), np.uint8)
    x = np.zeros((1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.matmul_gs(I8, w, np.zeros((2, 1), np.float32), 2, x)   # needs 2 groups
    with pytest.raises(ValueError):
        oracle.matmul_gs(I8, w, np.zeros((2, 4), np.float32), 0, x)   # gs < 1
