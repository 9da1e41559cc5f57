"""Seeded synthetic inputs for the quantized matmul workloads.

Shared by the tests, the smoke check and the benchmark: both the CPU oracle
and the HIP path are fed from here. This module only draws random bytes,
scales and activations with numpy's PCG64; it holds none of the matmul's
arithmetic (no dequantization, no packing rule, no sums).

Distributions (one scale per output row, activations N(0,1)):

  tiny        [O=256, I=512], S=1; int8 bytes uniform in [-127,127], scales
              U[0.001,0.02]; the same shape in f32, int4 and int2 (codes
              uniform over the whole code range, i.e. packed bytes uniform).
  dense_gemv  int4 [12288, 6144], S=1, scales U[0.002,0.05].
  moe_decode  8 experts x {gate int4 [2048,6144], up int4 [2048,6144],
              down int4 [6144,2048]}, S=1, scales U[0.002,0.05]; per expert
              one activation row for gate/up and its own row for down.
  int2_gemv   int2 [16384, 8192], S in {1,4,8}, scales U[0.01,0.1].
  prefill     int8 [6144, 6144], bytes = clip(rint(N(0,40)), -127, 127),
              scales U[0.001,0.01], S=512.

Seeds: 20261200 + workload number (tiny=1 ... prefill=5); sub-cases (format,
expert, S) add multiples of 100.
"""
from __future__ import annotations

import numpy as np

F32, I8, I4, I2 = 0, 1, 2, 3
BITS = {F32: 32, I8: 8, I4: 4, I2: 2}

WORKLOADS = {
    "tiny": 1,
    "dense_gemv": 2,
    "moe_decode": 3,
    "int2_gemv": 4,
    "prefill": 5,
}


def seed_for(workload: str, sub: int = 0) -> int:
    return 20261200 + WORKLOADS[workload] + 100 * sub


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def packed_row_bytes(fmt: int, I: int) -> int:
    """Storage size of one row: ceil(I * bits / 8) bytes."""
    return (I * BITS[fmt] + 7) // 8


def random_bytes(g: np.random.Generator, O: int, rb: int) -> np.ndarray:
    """Uniform bytes 0..255: every packed int4/int2 code uniform and independent."""
    return g.integers(0, 256, size=(O, rb), dtype=np.uint8)


def int8_uniform(g: np.random.Generator, O: int, I: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    return g.integers(lo, hi + 1, size=(O, I), dtype=np.int16).astype(np.int8).view(np.uint8)


def int8_rounded_normal(g: np.random.Generator, O: int, I: int, sigma: float = 40.0) -> np.ndarray:
    v = np.clip(np.rint(g.normal(0.0, sigma, size=(O, I))), -127, 127)
    return v.astype(np.int8).view(np.uint8)


def f32_normal(g: np.random.Generator, O: int, I: int) -> np.ndarray:
    return g.standard_normal((O, I), dtype=np.float32).view(np.uint8).reshape(O, 4 * I)


def f32_from_int8(w_i8: np.ndarray) -> np.ndarray:
    """f32 weights holding the same small integers as an int8 draw (exact)."""
    return w_i8.view(np.int8).astype(np.float32).view(np.uint8).reshape(w_i8.shape[0], -1)


def scales(g: np.random.Generator, O: int, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, O).astype(np.float32)


def group_scales(p, gs: int, lo: float, hi: float) -> np.ndarray:
    """One scale per (output row, group of gs columns) for problem p: float32 [O, ceil(I/gs)]."""
    g = rng(20261290 + gs + p.O)
    return g.uniform(lo, hi, size=(p.O, -(-p.I // gs))).astype(np.float32)


def activations(g: np.random.Generator, S: int, I: int) -> np.ndarray:
    return g.standard_normal((S, I), dtype=np.float32)


def weights(g: np.random.Generator, fmt: int, O: int, I: int) -> np.ndarray:
    """Packed [O, rb] weight bytes with codes uniform over the format's range."""
    if fmt == F32:
        return f32_normal(g, O, I)
    if fmt == I8:
        return int8_uniform(g, O, I)
    return random_bytes(g, O, packed_row_bytes(fmt, I))


class Problem:
    """One weight tensor plus activations: fmt, O, I, w bytes, scales, x [S, I]."""

    def __init__(self, name, fmt, O, I, w, sc, x):
        self.name, self.fmt, self.O, self.I = name, fmt, O, I
        self.w, self.scales, self.x = w, sc, x

    @property
    def S(self):
        return self.x.shape[0]

    @property
    def weight_bytes(self):
        return self.O * packed_row_bytes(self.fmt, self.I)


def tiny(fmt: int, S: int = 1, f32_variant: str = "normal") -> Problem:
    """The 256 x 512 check in one format (f32_variant: 'normal' or 'int8')."""
    O, I = 256, 512
    g = rng(seed_for("tiny", fmt))
    if fmt == F32 and f32_variant == "int8":
        g8 = rng(seed_for("tiny", I8))
        w = f32_from_int8(int8_uniform(g8, O, I))
    else:
        w = weights(g, fmt, O, I)
    sc = scales(g, O, 0.001, 0.02)
    x = activations(g, S, I)
    return Problem("tiny_%d" % fmt, fmt, O, I, w, sc, x)


def dense_gemv(S: int = 1) -> Problem:
    O, I = 12288, 6144
    g = rng(seed_for("dense_gemv"))
    w = random_bytes(g, O, packed_row_bytes(I4, I))
    sc = scales(g, O, 0.002, 0.05)
    x = activations(g, S, I)
    return Problem("dense_gemv", I4, O, I, w, sc, x)


def moe_decode(n_experts: int = 8, S: int = 1, hidden: int = 6144, inter: int = 2048):
    """List of 3*n_experts problems: per expert gate, up (shared x row) and down."""
    out = []
    for e in range(n_experts):
        g = rng(seed_for("moe_decode", e))
        x_gu = activations(g, S, hidden)
        x_dn = activations(g, S, inter)
        for name, O, I, x in (("gate", inter, hidden, x_gu), ("up", inter, hidden, x_gu),
                              ("down", hidden, inter, x_dn)):
            w = random_bytes(g, O, packed_row_bytes(I4, I))
            sc = scales(g, O, 0.002, 0.05)
            out.append(Problem("e%d_%s" % (e, name), I4, O, I, w, sc, x))
    return out


def int2_gemv(S: int = 1) -> Problem:
    O, I = 16384, 8192
    g = rng(seed_for("int2_gemv"))
    w = random_bytes(g, O, packed_row_bytes(I2, I))
    sc = scales(g, O, 0.01, 0.1)
    gx = rng(seed_for("int2_gemv", S))
    x = activations(gx, S, I)
    return Problem("int2_gemv_s%d" % S, I2, O, I, w, sc, x)


def prefill(S: int = 512) -> Problem:
    O, I = 6144, 6144
    g = rng(seed_for("prefill"))
    w = int8_rounded_normal(g, O, I)
    sc = scales(g, O, 0.001, 0.01)
    x = activations(g, S, I)
    return Problem("prefill", I8, O, I, w, sc, x)


def ragged(fmt: int, O: int, I: int, S: int, seed: int, scale_lo=0.001, scale_hi=0.05) -> Problem:
    """Arbitrary-shape case for edge tests (odd I, ragged O); padding bits random."""
    g = rng(seed)
    w = weights(g, fmt, O, I)
    sc = scales(g, O, scale_lo, scale_hi)
    x = activations(g, S, I)
    return Problem("ragged_%d_%dx%dx%d" % (fmt, O, I, S), fmt, O, I, w, sc, x)
