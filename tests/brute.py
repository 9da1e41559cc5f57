"""Exact-arithmetic brute force for tiny quantized matmuls (test helper).

Independent of the oracle: it reads a packed row as one little-endian bit
stream (element i of a b-bit format occupies stream bits [b*i, b*i + b)),
which is the low-nibble-first / low-bits-first packing stated for the int4
and int2 formats, and it does every product and sum in exact rational
arithmetic (fractions.Fraction). The exact result is then rounded once to
float32, round-to-nearest-even.

Dequant offsets follow colibri-analysis "CUDA 后端", section 1 (weight_at):
int4 subtracts 8, int2 subtracts 2, int8 is a signed byte.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np

F32, I8, I4, I2 = 0, 1, 2, 3
_BITS = {I8: 8, I4: 4, I2: 2}
_OFFSET = {I8: 0, I4: 8, I2: 2}


def codes(fmt: int, row: bytes, I: int) -> list:
    """Signed integer (or exact float) values of the first I elements of a row."""
    row = bytes(row)
    if fmt == F32:
        return [Fraction(struct.unpack("<f", row[4 * i:4 * i + 4])[0]) for i in range(I)]
    b = _BITS[fmt]
    stream = "".join(format(byte, "08b")[::-1] for byte in row)  # LSB of byte 0 first
    out = []
    for i in range(I):
        field = stream[b * i:b * i + b][::-1]  # back to MSB-first for int()
        v = int(field, 2)
        if fmt == I8:
            v = v - 256 if v >= 128 else v
        else:
            v -= _OFFSET[fmt]
        out.append(Fraction(v))
    return out


def round_to_f32(q: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    if q == 0:
        return np.float32(0.0)
    guess = np.float32(float(q))  # within an ulp of the answer
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)  # prefer even mantissa on ties
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def matmul_exact(fmt: int, w: np.ndarray, scales, x: np.ndarray, I: int):
    """Exact y[s,o] (Fractions) for packed rows w [O, >=rb], scales [O] or None, x [S, I]."""
    O = w.shape[0]
    S = x.shape[0]
    xs = [[Fraction(float(v)) for v in x[s]] for s in range(S)]
    out = [[None] * O for _ in range(S)]
    for o in range(O):
        q = codes(fmt, w[o].tobytes(), I)
        sc = Fraction(1) if scales is None else Fraction(float(scales[o]))
        for s in range(S):
            out[s][o] = sc * sum((q[i] * xs[s][i] for i in range(I)), Fraction(0))
    return out


def bound_exact(fmt: int, w: np.ndarray, scales, x: np.ndarray, I: int):
    """Exact A[s,o] = sum_i |scale[o] * q[o,i] * x[s,i]| (Fractions), the magnitude the
    acceptance bound 1e-5 * A + 1e-30 is stated against; written term by term
    from the same bit-stream codes, independently of the oracle."""
    O = w.shape[0]
    S = x.shape[0]
    xs = [[Fraction(float(v)) for v in x[s]] for s in range(S)]
    out = [[None] * O for _ in range(S)]
    for o in range(O):
        q = codes(fmt, w[o].tobytes(), I)
        sc = Fraction(1) if scales is None else Fraction(float(scales[o]))
        for s in range(S):
            out[s][o] = sum((abs(sc * q[i] * xs[s][i]) for i in range(I)), Fraction(0))
    return out


def matmul_rounded(fmt: int, w, scales, x, I: int) -> np.ndarray:
    ex = matmul_exact(fmt, w, scales, x, I)
    return np.array([[round_to_f32(v) for v in row] for row in ex], dtype=np.float32)


def matmul_gs_exact(fmt: int, w: np.ndarray, gscales: np.ndarray, gs: int, x: np.ndarray, I: int):
    """Exact y[s,o] with one scale per (row, group of gs columns): gscales [O, ceil(I/gs)]."""
    O = w.shape[0]
    S = x.shape[0]
    xs = [[Fraction(float(v)) for v in x[s]] for s in range(S)]
    out = [[None] * O for _ in range(S)]
    for o in range(O):
        q = codes(fmt, w[o].tobytes(), I)
        sc = [Fraction(float(v)) for v in gscales[o]]
        for s in range(S):
            out[s][o] = sum((sc[i // gs] * q[i] * xs[s][i] for i in range(I)), Fraction(0))
    return out


def bound_gs_exact(fmt: int, w: np.ndarray, gscales: np.ndarray, gs: int, x: np.ndarray, I: int):
    """Exact A[s,o] = sum_i |gscales[o, i // gs] * q[o,i] * x[s,i]| (Fractions)."""
    O = w.shape[0]
    S = x.shape[0]
    xs = [[Fraction(float(v)) for v in x[s]] for s in range(S)]
    out = [[None] * O for _ in range(S)]
    for o in range(O):
        q = codes(fmt, w[o].tobytes(), I)
        sc = [Fraction(float(v)) for v in gscales[o]]
        for s in range(S):
            out[s][o] = sum((abs(sc[i // gs] * q[i] * xs[s][i]) for i in range(I)), Fraction(0))
    return out


def matmul_gs_rounded(fmt: int, w, gscales, gs: int, x, I: int) -> np.ndarray:
    ex = matmul_gs_exact(fmt, w, gscales, gs, x, I)
    return np.array([[round_to_f32(v) for v in row] for row in ex], dtype=np.float32)
