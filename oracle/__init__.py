"""CPU oracle for the weight-only quantized matmul.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product library never imports,
links or runs it, and it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double accumulation,
one final rounding to float); this module compiles it with gcc and wraps it
with numpy arrays. What it computes is

    y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]

as given by the qmatmul.comp header quoted in colibri "第 8 章 · 02
CUDA/Metal/Vulkan 三后端" (section 四) and the weight_at / quant_matmul
description in colibri-analysis "CUDA 后端" (section 1). The readings the
pages leave open are listed at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, I8, I4, I2 = 0, 1, 2, 3
FMT_NAMES = {F32: "f32", I8: "i8", I4: "i4", I2: "i2"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # The mutation test points this at a deliberately broken copy of the
        # oracle to show that the pin suite rejects it.
        path = os.environ.get("ORACLE_LIB_UNDER_TEST")
        if not path:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        lib = ctypes.CDLL(path)
        lib.oracle_row_bytes.restype = ctypes.c_long
        lib.oracle_row_bytes.argtypes = [ctypes.c_int, ctypes.c_long]
        lib.oracle_weight.restype = ctypes.c_double
        lib.oracle_weight.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_matmul.restype = ctypes.c_int
        lib.oracle_matmul.argtypes = [
            ctypes.c_int, ctypes.c_long, ctypes.c_long, ctypes.c_void_p, ctypes.c_long,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int]
        if hasattr(lib, "oracle_silu_mul"):
            lib.oracle_silu_mul.restype = None
            lib.oracle_silu_mul.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
        if hasattr(lib, "oracle_matmul_gs"):
            lib.oracle_matmul_gs.restype = ctypes.c_int
            lib.oracle_matmul_gs.argtypes = [
                ctypes.c_int, ctypes.c_long, ctypes.c_long, ctypes.c_void_p, ctypes.c_long,
                ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def row_bytes(fmt: int, I: int) -> int:
    rb = _load().oracle_row_bytes(int(fmt), int(I))
    if rb < 0:
        raise ValueError("invalid fmt/I: %r/%r" % (fmt, I))
    return int(rb)


def dequant_row(fmt: int, row: np.ndarray, I: int) -> np.ndarray:
    """Dequantized values (float64) of the first I elements of one packed row."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    if row.size < row_bytes(fmt, I):
        raise ValueError("row too short")
    lib = _load()
    p = row.ctypes.data
    return np.array([lib.oracle_weight(int(fmt), p, i) for i in range(I)], dtype=np.float64)


def matmul(fmt: int, w: np.ndarray, scales, x: np.ndarray, I: int | None = None,
           threads: int | None = None, want_bound: bool = True):
    """Oracle y (float32 [S,O]) and bound magnitude A (float64 [S,O]).

    w: uint8 [O, row_stride] packed rows (row_stride >= row_bytes(fmt, I)).
    scales: float32 [O] or None (f32 only: scale 1).
    x: float32 [S, I].
    """
    lib = _load()
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [S, I]")
    S = x.shape[0]
    if I is None:
        I = x.shape[1]
    if x.shape[1] != I:
        raise ValueError("x has %d columns, I=%d" % (x.shape[1], I))
    if w.ndim != 2:
        raise ValueError("w must be [O, row_stride] bytes")
    O, stride = w.shape
    if scales is not None:
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        if scales.shape != (O,):
            raise ValueError("scales must be [O]")
    y = np.empty((S, O), dtype=np.float32)
    a = np.empty((S, O), dtype=np.float64) if want_bound else None
    rc = lib.oracle_matmul(
        int(fmt), O, int(I), w.ctypes.data, stride,
        scales.ctypes.data if scales is not None else None,
        x.ctypes.data, S, y.ctypes.data, a.ctypes.data if a is not None else None,
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_matmul rejected its arguments (rc=%d)" % rc)
    return y, a


def matmul_rows(fmt: int, w: np.ndarray, scales, x: np.ndarray, rows, I: int | None = None,
                threads: int | None = None):
    """Oracle y and A restricted to output rows ``rows`` (columns of y): [S, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    sub_w = np.ascontiguousarray(np.asarray(w)[rows])
    sub_s = None if scales is None else np.ascontiguousarray(np.asarray(scales)[rows])
    return matmul(fmt, sub_w, sub_s, x, I=I, threads=threads)


def n_groups(I: int, gs: int) -> int:
    return (int(I) + int(gs) - 1) // int(gs)


def matmul_gs(fmt: int, w: np.ndarray, scales: np.ndarray, gs: int, x: np.ndarray, I: int | None = None,
              threads: int | None = None, want_bound: bool = True):
    """Oracle with group-wise scales: y (float32 [S,O]) and bound magnitude A.

    scales: float32 [O, ceil(I/gs)], one scale per (row, group of gs columns).
    """
    lib = _load()
    if int(gs) < 1:
        raise ValueError("gs must be >= 1")
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [S, I]")
    S = x.shape[0]
    if I is None:
        I = x.shape[1]
    if x.shape[1] != I:
        raise ValueError("x has %d columns, I=%d" % (x.shape[1], I))
    O, stride = w.shape
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if scales.shape != (O, n_groups(I, gs)):
        raise ValueError("scales must be [O, ceil(I/gs)]")
    y = np.empty((S, O), dtype=np.float32)
    a = np.empty((S, O), dtype=np.float64) if want_bound else None
    rc = lib.oracle_matmul_gs(
        int(fmt), O, int(I), w.ctypes.data, stride, scales.ctypes.data, int(gs),
        x.ctypes.data, S, y.ctypes.data, a.ctypes.data if a is not None else None,
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_matmul_gs rejected its arguments (rc=%d)" % rc)
    return y, a


def matmul_gs_rows(fmt: int, w: np.ndarray, scales: np.ndarray, gs: int, x: np.ndarray, rows,
                   I: int | None = None, threads: int | None = None):
    """matmul_gs restricted to output rows ``rows``: [S, len(rows)]."""
    rows = np.asarray(rows, dtype=np.int64)
    return matmul_gs(fmt, np.ascontiguousarray(np.asarray(w)[rows]),
                     np.ascontiguousarray(np.asarray(scales)[rows]), gs, x, I=I, threads=threads)


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = fl32(silu(g) * u) elementwise, computed in double (float32 in, float32 out)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    h = np.empty_like(g)
    _load().oracle_silu_mul(g.ctypes.data, u.ctypes.data, g.size, h.ctypes.data)
    return h


def swiglu_ffn(fmt: int, gate, up, down, x: np.ndarray):
    """One expert's feed-forward step, every stage from the oracle.

    gate, up: (w, scales) of [O, I] tensors; down: (w, scales) of an [I2, O]
    tensor; x: float32 [S, I]. Returns a dict with g, u (and their bound
    magnitudes Ag, Au), h = silu_mul(g, u), y = down . h (and Ay).
    """
    g, ag = matmul(fmt, gate[0], gate[1], x)
    u, au = matmul(fmt, up[0], up[1], x)
    h = silu_mul(g, u)
    y, ay = matmul(fmt, down[0], down[1], h)
    return {"g": g, "Ag": ag, "u": u, "Au": au, "h": h, "y": y, "Ay": ay}
