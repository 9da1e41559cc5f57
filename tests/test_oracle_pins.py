"""Pins for the CPU oracle: it is checked against things other than itself.

- hand-decoded bytes and hand-worked matmuls (tests/golden/);
- exact rational brute force on tiny shapes (tests/brute.py);
- exhaustive code tables through one-hot activations;
- closed forms and invariants: zero scale, all-zero-code rows, integer
  activations, power-of-two linearity, cross-format equality, row
  independence, thread-count independence, padding bits ignored;
- numpy's float64 matmul for f32 weights without scales.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import brute
import golden_io
import oracle
import packing
import synth

F32, I8, I4, I2 = 0, 1, 2, 3
ALL = (F32, I8, I4, I2)
RANGE = {I8: (-127, 127), I4: (-8, 7), I2: (-2, 1)}


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)
    return np.abs(a - b) / sp


# --------------------------------------------------------------------------------------
# golden fixtures


@pytest.mark.parametrize("case", golden_io.dequant_table(), ids=lambda c: "%d-%s" % (c[0], c[1].hex()))
def test_dequant_table(case):
    fmt, raw, vals = case
    row = np.frombuffer(raw, dtype=np.uint8)
    got = oracle.dequant_row(fmt, row, len(vals))
    np.testing.assert_array_equal(got, np.array(vals))
    assert [float(v) for v in brute.codes(fmt, raw, len(vals))] == vals


@pytest.mark.parametrize("case", golden_io.dequant_table(), ids=lambda c: "%d-%s" % (c[0], c[1].hex()))
def test_packer_reproduces_table(case):
    fmt, raw, vals = case
    packed = packing.pack(fmt, np.array([vals]))
    assert packed.tobytes() == raw


@pytest.mark.parametrize("case", golden_io.worked_examples(), ids=lambda c: c["name"])
def test_worked_examples(case):
    y, a = oracle.matmul(case["fmt"], case["w"], case["scales"], case["x"], I=case["I"])
    np.testing.assert_array_equal(y, case["y"])
    np.testing.assert_array_equal(a, case["A"])  # hand-worked bound magnitudes (exact)
    yb = brute.matmul_rounded(case["fmt"], case["w"], case["scales"], case["x"], case["I"])
    np.testing.assert_array_equal(yb, case["y"])
    ab = brute.bound_exact(case["fmt"], case["w"], case["scales"], case["x"], case["I"])
    np.testing.assert_array_equal(np.array([[float(v) for v in r] for r in ab]), case["A"])


# --------------------------------------------------------------------------------------
# brute force


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("shape", [(3, 7, 1), (5, 16, 2), (8, 33, 3), (2, 64, 1)])
def test_brute_force(fmt, shape):
    O, I, S = shape
    g = synth.rng(1000 + 10 * fmt + O)
    w = synth.weights(g, fmt, O, I)
    sc = synth.scales(g, O, 0.001, 0.05)
    x = synth.activations(g, S, I)
    y, a = oracle.matmul(fmt, w, sc, x)
    yb = brute.matmul_rounded(fmt, w, sc, x, I)
    d = ulp_diff(y, yb)
    assert d.max() <= 1.0, d.max()
    assert np.mean(d == 0) >= 0.9


def rel_to_exact(a: np.ndarray, exact) -> float:
    """Largest |a - exact| / exact over the entries (0 where both are 0)."""
    worst = 0.0
    for s, row in enumerate(exact):
        for o, v in enumerate(row):
            d = abs(Fraction(float(a[s, o])) - v)
            if v == 0:
                assert d == 0, (s, o, float(a[s, o]))
            else:
                worst = max(worst, float(d / v))
    return worst


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("shape", [(3, 7, 1), (5, 16, 2), (8, 33, 3), (2, 64, 1)])
def test_bound_magnitude_brute_force(fmt, shape):
    """A = sum_i |scale q x| against exact rationals: every parity tolerance is 1e-5 * A + 1e-30,
    so A itself needs a pin. The oracle sums |q x| in double (n terms, each exact): relative
    error <= n * 2^-53, far inside 1e-12."""
    O, I, S = shape
    g = synth.rng(1000 + 10 * fmt + O)
    w = synth.weights(g, fmt, O, I)
    sc = synth.scales(g, O, 0.001, 0.05)
    x = synth.activations(g, S, I)
    _, a = oracle.matmul(fmt, w, sc, x)
    assert rel_to_exact(a, brute.bound_exact(fmt, w, sc, x, I)) <= 1e-12


def test_bound_magnitude_signs_and_zero_codes():
    """Mixed signs in q, x and the scale (a negative scale is |scale|): A is the sum of the
    magnitudes, not the magnitude of the sum; zero-point codes add nothing to it."""
    vals = np.array([[-2, 1, 0, -1, 1, 0, -2, 1], [0, 0, 0, 0, 0, 0, 0, 1]])
    x = np.array([[1.5, -2.0, 7.0, 0.25, -4.0, 3.0, -0.5, 1.0]], np.float32)
    for fmt in (I8, I4, I2):
        w = packing.pack(fmt, vals)
        sc = np.array([-0.5, 2.0], np.float32)
        y, a = oracle.matmul(fmt, w, sc, x)
        # row 0: |q x| = 3 + 2 + 0 + 0.25 + 4 + 0 + 1 + 1 = 11.25 ; row 1: 1
        np.testing.assert_array_equal(a, [[5.625, 2.0]])
        # signed sum: -3 - 2 + 0 - 0.25 - 4 + 0 + 1 + 1 = -7.25 -> * -0.5
        np.testing.assert_array_equal(y, np.array([[3.625, 2.0]], np.float32))
        ab = brute.bound_exact(fmt, w, sc, x, 8)
        assert [float(v) for v in ab[0]] == [5.625, 2.0]


def test_brute_force_f32_without_scales():
    g = synth.rng(4242)
    w = synth.weights(g, F32, 4, 9)
    x = synth.activations(g, 2, 9)
    y, _ = oracle.matmul(F32, w, None, x)
    yb = brute.matmul_rounded(F32, w, None, x, 9)
    assert ulp_diff(y, yb).max() <= 1.0


# --------------------------------------------------------------------------------------
# exhaustive codes via one-hot activations


@pytest.mark.parametrize("fmt,I", [(I8, 256), (I4, 512), (I2, 1024)])
def test_exhaustive_codes_one_hot(fmt, I):
    row = np.arange(256, dtype=np.uint8)[None, :]  # every byte value once
    w = np.repeat(row, 3, axis=0)
    sc = np.array([1.0, 0.0137, 3.5], dtype=np.float32)
    q = np.array([float(v) for v in brute.codes(fmt, row[0].tobytes(), I)])
    # pick a spread of columns including the first/last element of a byte
    cols = sorted(set(list(range(0, I, max(1, I // 64))) + list(range(min(I, 16))) + [I - 1]))
    x = np.zeros((len(cols), I), dtype=np.float32)
    for s, c in enumerate(cols):
        x[s, c] = 1.0
    y, _ = oracle.matmul(fmt, w, sc, x)
    for s, c in enumerate(cols):
        expect = (sc.astype(np.float64) * q[c]).astype(np.float32)
        np.testing.assert_array_equal(y[s], expect)
    # the full code set appears: every value of the range is hit
    lo, hi = RANGE[fmt]
    assert set(q.astype(int)) == set(range(lo if fmt != I8 else -128, hi + 1))


def test_int8_full_byte_map():
    """All 256 int8 bytes: value = byte read as two's complement."""
    raw = bytes(range(256))
    got = oracle.dequant_row(I8, np.frombuffer(raw, np.uint8), 256)
    assert list(got[:128]) == list(range(128))
    assert list(got[128:]) == list(range(-128, 0))


# --------------------------------------------------------------------------------------
# closed forms and invariants


@pytest.mark.parametrize("fmt", ALL)
def test_zero_scale_gives_zero(fmt):
    p = synth.ragged(fmt, 17, 45, 3, seed=7)
    sc = p.scales.copy()
    sc[::3] = 0.0
    y, _ = oracle.matmul(fmt, p.w, sc, p.x)
    assert np.all(y[:, ::3] == 0.0)
    assert np.all(y[:, 1::3] != 0.0)


@pytest.mark.parametrize("fmt,byte", [(I8, 0x00), (I4, 0x88), (I2, 0xAA), (F32, 0x00)])
def test_zero_code_rows(fmt, byte):
    p = synth.ragged(fmt, 9, 40, 2, seed=11)
    w = p.w.copy()
    w[4, :] = byte
    y, a = oracle.matmul(fmt, w, p.scales, p.x)
    assert np.all(y[:, 4] == 0.0) and np.all(a[:, 4] == 0.0)
    assert np.all(y[:, 3] != 0.0)


@pytest.mark.parametrize("fmt", (I8, I4, I2))
def test_one_hot_selects_scaled_column(fmt):
    p = synth.ragged(fmt, 12, 37, 1, seed=13)
    q = np.array([[float(v) for v in brute.codes(fmt, p.w[o].tobytes(), p.I)] for o in range(p.O)])
    for col in (0, 1, 2, 3, 17, 36):
        x = np.zeros((1, p.I), np.float32)
        x[0, col] = 1.0
        y, _ = oracle.matmul(fmt, p.w, p.scales, x)
        np.testing.assert_array_equal(y[0], (p.scales.astype(np.float64) * q[:, col]).astype(np.float32))


@pytest.mark.parametrize("fmt", (I8, I4, I2))
def test_integer_activations_closed_form(fmt):
    """x = 1: y = fl32(scale * row sum of codes), an exact integer sum."""
    p = synth.ragged(fmt, 20, 301, 1, seed=17)
    q = np.array([[int(v) for v in brute.codes(fmt, p.w[o].tobytes(), p.I)] for o in range(p.O)])
    x = np.ones((1, p.I), np.float32)
    y, _ = oracle.matmul(fmt, p.w, p.scales, x)
    expect = (p.scales.astype(np.float64) * q.sum(axis=1)).astype(np.float32)
    np.testing.assert_array_equal(y[0], expect)


@pytest.mark.parametrize("fmt", ALL)
def test_power_of_two_linearity(fmt):
    p = synth.ragged(fmt, 15, 64, 2, seed=19)
    y1, _ = oracle.matmul(fmt, p.w, p.scales, p.x)
    for k in (-3, 1, 5):
        yk, _ = oracle.matmul(fmt, p.w, p.scales, (p.x * np.float32(2.0 ** k)).astype(np.float32))
        np.testing.assert_array_equal(yk, (y1 * np.float32(2.0 ** k)).astype(np.float32))


@pytest.mark.parametrize("fmt", ALL)
def test_linearity_within_bound(fmt):
    p = synth.ragged(fmt, 15, 64, 1, seed=23)
    g = synth.rng(99)
    x2 = synth.activations(g, 1, p.I)
    al, be = np.float32(0.75), np.float32(-1.25)
    xc = (al * p.x + be * x2).astype(np.float32)
    y1, a1 = oracle.matmul(fmt, p.w, p.scales, p.x)
    y2, a2 = oracle.matmul(fmt, p.w, p.scales, x2)
    yc, _ = oracle.matmul(fmt, p.w, p.scales, xc)
    lin = al * y1.astype(np.float64) + be * y2.astype(np.float64)
    bound = 1e-5 * (abs(al) * a1 + abs(be) * a2) + 1e-30
    assert np.all(np.abs(yc - lin) <= bound)


def test_cross_format_equality():
    g = synth.rng(31)
    O, I, S = 11, 29, 2
    vals = g.integers(-2, 2, size=(O, I))  # representable in every format
    sc = synth.scales(g, O, 0.01, 0.1)
    x = synth.activations(g, S, I)
    ys = [oracle.matmul(fmt, packing.pack(fmt, vals), sc, x)[0] for fmt in ALL]
    for y in ys[1:]:
        np.testing.assert_array_equal(y, ys[0])


@pytest.mark.parametrize("fmt", ALL)
def test_row_independence(fmt):
    p = synth.ragged(fmt, 10, 50, 4, seed=37)
    y, _ = oracle.matmul(fmt, p.w, p.scales, p.x)
    for s in range(p.S):
        ys, _ = oracle.matmul(fmt, p.w, p.scales, p.x[s:s + 1])
        np.testing.assert_array_equal(ys[0], y[s])


def test_f32_textbook_matmul():
    g = synth.rng(41)
    O, I, S = 23, 57, 3
    wf = g.standard_normal((O, I), dtype=np.float32)
    x = synth.activations(g, S, I)
    y, _ = oracle.matmul(F32, wf.view(np.uint8).reshape(O, 4 * I), None, x)
    ref = (x.astype(np.float64) @ wf.astype(np.float64).T).astype(np.float32)
    assert ulp_diff(y, ref).max() <= 1.0


def test_f32_null_scales_equal_unit_scales():
    p = synth.ragged(F32, 8, 21, 2, seed=43)
    y0, _ = oracle.matmul(F32, p.w, None, p.x)
    y1, _ = oracle.matmul(F32, p.w, np.ones(p.O, np.float32), p.x)
    np.testing.assert_array_equal(y0, y1)


@pytest.mark.parametrize("fmt", ALL)
def test_thread_count_independence(fmt):
    p = synth.ragged(fmt, 64, 130, 3, seed=47)
    y1, a1 = oracle.matmul(fmt, p.w, p.scales, p.x, threads=1)
    y8, a8 = oracle.matmul(fmt, p.w, p.scales, p.x, threads=8)
    np.testing.assert_array_equal(y1, y8)
    np.testing.assert_array_equal(a1, a8)


@pytest.mark.parametrize("fmt,I", [(I4, 7), (I4, 31), (I2, 5), (I2, 30), (I2, 33)])
def test_padding_bits_ignored(fmt, I):
    g = synth.rng(53 + I)
    O = 6
    lo, hi = RANGE[fmt]
    vals = g.integers(lo, hi + 1, size=(O, I))
    sc = synth.scales(g, O, 0.01, 0.1)
    x = synth.activations(g, 2, I)
    y0, _ = oracle.matmul(fmt, packing.pack(fmt, vals, pad_bits=0), sc, x)
    y1, _ = oracle.matmul(fmt, packing.pack(fmt, vals, pad_bits=0xF), sc, x)
    np.testing.assert_array_equal(y0, y1)


def test_row_stride_padding():
    p = synth.ragged(I4, 5, 19, 2, seed=59)
    wide = np.full((p.O, p.w.shape[1] + 13), 0x5A, dtype=np.uint8)
    wide[:, :p.w.shape[1]] = p.w
    y0, _ = oracle.matmul(I4, p.w, p.scales, p.x)
    y1, _ = oracle.matmul(I4, wide, p.scales, p.x, I=p.I)
    np.testing.assert_array_equal(y0, y1)


def test_bound_magnitude_dominates_result():
    p = synth.ragged(I4, 30, 200, 2, seed=61)
    y, a = oracle.matmul(I4, p.w, p.scales, p.x)
    assert np.all(a >= np.abs(y.astype(np.float64)) * (1 - 1e-7))


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.row_bytes(7, 10)
    p = synth.ragged(I8, 3, 8, 1, seed=67)
    with pytest.raises(ValueError):
        oracle.matmul(I8, p.w, None, p.x)  # quantized weights need scales


def test_row_bytes():
    assert [oracle.row_bytes(f, 9) for f in ALL] == [36, 9, 5, 3]
    assert [oracle.row_bytes(f, 8) for f in ALL] == [32, 8, 4, 2]
    assert oracle.row_bytes(I4, 0) == 0
