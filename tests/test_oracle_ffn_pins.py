"""Pins for the oracle's SiLU-gated product h = fl32(silu(g) * u),
silu(z) = z / (1 + e^-z): the reading taken for the activation between the
fused gate/up matmul and the down projection (colibri "第 8 章 · 02
CUDA/Metal/Vulkan 三后端", learning goals and section recap, name the gated
up-projection shader qmatmul_gate_up.comp but not its activation). Closed
forms, identities and limits, not a re-evaluation of the same formula."""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth


def ulps(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)
    return np.abs(a - b) / sp


def test_closed_forms():
    # sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so silu(+-ln 3) = +-ln 3 * (3/4 or 1/4)
    z = np.array([math.log(3.0), -math.log(3.0), math.log(7.0)], dtype=np.float32)
    u = np.array([1.0, 2.0, -0.5], dtype=np.float32)
    expect = np.array([0.75 * float(z[0]) * 1.0, 0.25 * float(z[1]) * 2.0, 0.875 * float(z[2]) * -0.5])
    assert ulps(oracle.silu_mul(z, u), expect).max() <= 1.0


def test_zero_and_gating():
    z = np.array([0.0, 0.0, 3.0, -3.0], dtype=np.float32)
    u = np.array([5.0, -7.0, 0.0, 0.0], dtype=np.float32)
    h = oracle.silu_mul(z, u)
    assert np.all(h == 0.0)


def test_odd_part_identity():
    # silu(z) - silu(-z) = z * (sigma(z) + sigma(-z)) = z
    z = np.linspace(-20, 20, 401).astype(np.float32)
    one = np.ones_like(z)
    d = oracle.silu_mul(z, one).astype(np.float64) - oracle.silu_mul(-z, one).astype(np.float64)
    tol = 2 * np.spacing(np.abs(z).astype(np.float32)).astype(np.float64) + 1e-30
    assert np.all(np.abs(d - z.astype(np.float64)) <= tol)


def test_limits():
    big = np.array([40.0, 80.0, 1000.0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.silu_mul(big, np.ones_like(big)), big)  # sigma rounds to 1
    neg = np.array([-30.0, -60.0, -100.0], dtype=np.float32)
    h = oracle.silu_mul(neg, np.ones_like(neg))
    assert np.all(h <= 0) and np.all(np.abs(h) <= 1e-11 * np.abs(neg))
    # minimum of silu: about -0.2785 near z = -1.2785
    zz = np.linspace(-3, 0, 3001).astype(np.float32)
    assert abs(float(oracle.silu_mul(zz, np.ones_like(zz)).min()) + 0.27846) < 1e-4


def test_ffn_chain_with_zero_gate_gives_zero():
    fmt, O, I, I2 = 1, 16, 64, 32
    g = synth.rng(3600)
    zero_gate = np.zeros((O, I), np.uint8)        # int8 codes 0: g = 0, so h = 0
    up = synth.weights(g, fmt, O, I)
    down = synth.weights(g, fmt, I2, O)
    sc = synth.scales(g, O, 0.01, 0.1)
    sd = synth.scales(g, I2, 0.01, 0.1)
    x = synth.activations(g, 3, I)
    r = oracle.swiglu_ffn(fmt, (zero_gate, sc), (up, sc), (down, sd), x)
    assert np.all(r["g"] == 0) and np.all(r["h"] == 0) and np.all(r["y"] == 0)
