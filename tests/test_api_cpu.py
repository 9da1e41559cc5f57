"""C-ABI checks that need no GPU: exports, argument validation, plans, status strings."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import weight_only_quantized_matmul_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wqmm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("wq_init", "wq_mem_info", "wq_tensor_upload", "wq_matmul", "wq_matmul_t",
                 "wq_matmul_dev", "wq_grouped_create", "wq_grouped_matmul_dev", "wq_grouped_free",
                 "wq_tensor_free", "wq_strerror", "wq_swiglu_create", "wq_swiglu_matmul_dev",
                 "wq_swiglu_ffn_dev"):
        assert must in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", wq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (wq_[a-z_]+)\b", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(wq.lib, n)


def test_header_compiles_as_c_and_links():
    prog = r'''
#include "wqmm.h"
#include <stdio.h>
int main(void) {
    int (*fns[])(void) = {0};
    (void)fns;
    printf("%ld %s\n", wq_row_bytes(WQ_I4, 7), wq_strerror(WQ_E_MISMATCH));
    return 0;
}
'''
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "t.c")
        exe = os.path.join(tmp, "t")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), c,
                        "-o", exe, wq.LIB_PATH, "-Wl,-rpath," + os.path.dirname(wq.LIB_PATH)],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
        assert out.split()[0] == "4"


def test_strerror_covers_every_code():
    codes = [wq.WQ_OK, wq.WQ_E_INVAL, wq.WQ_E_NODEV, wq.WQ_E_NOTINIT, wq.WQ_E_OOM,
             wq.WQ_E_MISMATCH, wq.WQ_E_HIP, wq.WQ_E_FAULT, wq.WQ_E_UNSUPPORTED]
    texts = [wq.wq_strerror(c) for c in codes]
    assert all(texts) and len(set(texts)) == len(texts)
    assert "unknown" in wq.wq_strerror(12345)


def test_row_bytes():
    assert [wq.wq_row_bytes(f, 9) for f in range(4)] == [36, 9, 5, 3]
    assert wq.wq_row_bytes(7, 9) == -1
    assert wq.wq_row_bytes(wq.WQ_I4, -1) == -1


def _plan(fmt, O, I, S):
    s = wq.wq_describe_plan(fmt, O, I, S)
    kind, *kv = s.split()
    return kind, dict(item.split("=") for item in kv)


import contextlib


@contextlib.contextmanager
def forced(**env):
    """WQ_* knobs for host-only plan queries: wq_init reads them before it looks for a
    device (and fails here, having none)."""
    old = {k: os.environ.get(k) for k in env}
    try:
        for k, v in env.items():
            os.environ[k] = v
        wq.lib.wq_init(None, 0)
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        wq.lib.wq_init(None, 0)


@pytest.mark.parametrize("fmt,O,I,S", [
    (wq.WQ_I4, 12288, 6144, 1), (wq.WQ_I2, 16384, 8192, 1), (wq.WQ_I4, 2048, 6144, 1), (wq.WQ_I4, 6144, 2048, 1),
    (wq.WQ_I8, 256, 512, 1), (wq.WQ_F32, 256, 512, 1), (wq.WQ_F32, 256, 512, 4),
    # rows the matrix-core few-rows kernel cannot read in 16-byte runs (I % 4 != 0)
    (wq.WQ_I8, 7, 33, 5), (wq.WQ_F32, 1, 1, 1), (wq.WQ_I2, 3, 5, 2), (wq.WQ_F32, 100, 3000, 8),
    (wq.WQ_I4, 255, 511, 3), (wq.WQ_I8, 255, 513, 8),
])
def test_gemv_plan_invariants(fmt, O, I, S):
    kind, p = _plan(fmt, O, I, S)
    assert kind == "gemv"
    p = {k: int(v) for k, v in p.items()}
    stride = -(-wq.wq_row_bytes(fmt, I) // 16) * 16
    assert p["smax"] >= S and p["smax"] in (1, 2, 4, 8)
    assert 1 <= p["team"] <= 8 and p["block"] <= 512 and p["block"] % 64 == 0
    assert 1 <= p["k"] <= p["kmax"]
    assert 64 * p["lw"] * p["team"] * p["k"] >= stride          # every byte of a row is covered
    assert 64 * p["lw"] * p["team"] * (p["k"] - 1) < stride     # no empty slot
    teams = p["grid"] * p["block"] // (64 * p["team"])
    assert teams * p["rows_per_team"] >= O                      # every row is owned
    assert (p["grid"] - 1) * p["block"] // (64 * p["team"]) * p["rows_per_team"] < O  # no idle block
    assert p["rows_per_team"] % p["d"] == 0


def test_headline_plan_shape():
    kind, p = _plan(wq.WQ_I4, 12288, 6144, 1)
    assert kind == "gemv" and p["team"] == "1" and p["k"] == "3" and p["lw"] == "16"


@pytest.mark.parametrize("fmt,O,I,S", [
    (wq.WQ_I4, 12288, 6144, 2), (wq.WQ_I4, 12288, 6144, 8), (wq.WQ_I2, 16384, 8192, 4), (wq.WQ_I2, 16384, 8192, 8),
    (wq.WQ_I2, 16384, 8192, 16), (wq.WQ_I8, 6144, 6144, 8), (wq.WQ_I8, 6144, 6144, 16), (wq.WQ_I4, 2048, 6144, 4),
    (wq.WQ_I4, 256, 512, 3), (wq.WQ_I2, 3, 8, 2), (wq.WQ_I8, 100, 4, 11),
    (wq.WQ_I4, 12288, 6144, 17), (wq.WQ_I4, 12288, 6144, 24), (wq.WQ_I4, 12288, 6144, 32),
    (wq.WQ_I2, 16384, 8192, 20), (wq.WQ_I8, 6144, 6144, 25), (wq.WQ_I4, 100, 300, 31), (wq.WQ_I2, 5000, 1000, 22),
])
def test_skinny_plan_invariants(fmt, O, I, S):
    """2 <= S <= 32 on quantized rows read in 16-byte runs: the matrix-core few-rows kernel.
    Every output row is owned by a block, every 128-position chunk of a row by a wave,
    the stacked activation parts (3 S rows) fit the plan's MFMA fragments and every
    lane's activation runs cover the 4 S runs of a chunk."""
    kind, p = _plan(fmt, O, I, S)
    assert kind == "skinny", (kind, p)
    p = {k: int(v) for k, v in p.items()}
    m_want = 1 if S <= 5 else 2 if S <= 10 else 3 if S <= 16 else 4 if S <= 20 else 5 if S <= 24 else 6
    assert p["m"] == m_want and 3 * S <= 16 * p["m"]
    assert 16 * p["rpl"] >= 4 * S and (S > 16 or p["rpl"] == -(-S // 4))
    assert p["grid"] * 16 * p["nb"] >= O and (p["grid"] - 1) * 16 * p["nb"] < O
    stride = -(-wq.wq_row_bytes(fmt, I) // 16) * 16
    fields = stride * {wq.WQ_I8: 1, wq.WQ_I4: 2, wq.WQ_I2: 4}[fmt]
    assert p["chunks"] * 128 >= fields and p["chunks"] % 2 == 0
    assert p["waves"] * p["chunks_per_wave"] >= p["chunks"] and p["chunks_per_wave"] % 2 == 0
    assert p["ring"] in (2, 4, 6)
    assert p["block"] == 64 * p["waves"] <= 1024 and p["workspace"] == 0
    if S <= 16:  # 16-wave blocks only with at most two fragments (registers)
        assert p["waves"] == 8 or p["m"] <= 2
    else:  # four waves: their operand buffers fit in LDS; one wave per SIMD holds the tiles
        assert p["waves"] == 4 and p["ring"] == 2 and 1 <= p["nb"] <= (3 if p["m"] == 6 else 4)
        # the fewest output blocks that keep one block per CU (m = 4 may take a second round)
        assert p["grid"] <= 256 or (p["m"] == 4 and p["nb"] == 4)
        assert p["nb"] == 1 or -(-(-(-O // 16)) // (p["nb"] - 1)) > 256


@pytest.mark.parametrize("fmt,O,I,S,kind", [(wq.WQ_I2, 16384, 8192, 24, "skinny"), (wq.WQ_I2, 16384, 8192, 32, "tiled"),
                                            (wq.WQ_I4, 60000, 2048, 20, "skinny"), (wq.WQ_I4, 60000, 2048, 21, "tiled"),
                                            (wq.WQ_I8, 6144, 6144, 32, "skinny")])
def test_wide_few_rows_kernel_or_tiled(fmt, O, I, S, kind):
    """Above S = 16 the few-rows kernel runs one 4-wave block per CU; where no compiled block
    size keeps the grid to one round (m >= 5: 3 or 4 output blocks), the tiled kernel takes it."""
    assert _plan(fmt, O, I, S)[0] == kind


def test_skinny_plan_fills_the_chip_for_the_small_s_workloads():
    for fmt, O, I in ((wq.WQ_I4, 12288, 6144), (wq.WQ_I2, 16384, 8192)):
        for S in (2, 4, 8, 16):
            kind, p = _plan(fmt, O, I, S)
            assert kind == "skinny" and int(p["grid"]) >= 256 and int(p["waves"]) == 8, p
            if S <= 8:  # one block per CU
                assert int(p["grid"]) == 256, p


@pytest.mark.parametrize("fmt,O,I,S", [(wq.WQ_I8, 6144, 6144, 512), (wq.WQ_I4, 100, 200, 33),
                                       (wq.WQ_F32, 64, 300000, 8)])
def test_tiled_plan(fmt, O, I, S):
    kind, p = _plan(fmt, O, I, S)
    assert kind == "tiled"
    assert int(p["tiles_s"]) * int(p["bm"]) >= S and int(p["tiles_o"]) * int(p["bn"]) >= O
    ks = int(p["ksplit"])
    assert int(p["grid"]) == int(p["tiles_s"]) * int(p["tiles_o"]) * ks
    # plane rows hold every tile row the kernel reads: bm divides the 128-row padding
    assert 128 % int(p["bm"]) == 0 and 128 % int(p["bk"]) == 0
    if fmt == wq.WQ_F32:  # no planes; split K keeps fp32 partials per chunk
        assert p["mode"] == "fp32" and int(p["workspace"]) == (0 if ks == 1 else ks * S * O * 4)
    else:
        # three bf16 planes of round_up(S, 128) rows (16 for the 16-row tile) by round_up(fields per row, 128)
        stride = -(-wq.wq_row_bytes(fmt, I) // 16) * 16
        fields = stride * {wq.WQ_I8: 1, wq.WQ_I4: 2, wq.WQ_I2: 4}[fmt]
        assert p["mode"] == "bf16x3"
        sp_align = 16 if p["bm"] == "16" else 128
        planes = 3 * (-(-S // sp_align) * sp_align) * (-(-fields // 128) * 128) * 2
        if ks == 1:
            assert int(p["workspace"]) == planes
        else:  # split K: fp32 partials per chunk after the planes
            assert int(p["workspace"]) == -(-planes // 256) * 256 + ks * S * O * 4


@pytest.mark.parametrize("fmt,O,I,S,ks", [(wq.WQ_I4, 12288, 6144, 8, 6), (wq.WQ_I2, 16384, 8192, 12, 4),
                                          (wq.WQ_I4, 12288, 6144, 32, 8), (wq.WQ_I2, 16384, 8192, 40, 2),
                                          (wq.WQ_I8, 6144, 6144, 512, 1), (wq.WQ_I4, 100, 200, 9, 1),
                                          (wq.WQ_F32, 12288, 6144, 9, 3), (wq.WQ_F32, 64, 300000, 8, 512),
                                          (wq.WQ_F32, 4096, 4096, 200, 2), (wq.WQ_F32, 4096, 4096, 512, 3),
                                          (wq.WQ_F32, 16384, 4096, 512, 1)])
def test_tiled_split_k_plan(fmt, O, I, S, ks):
    """Few tiles split K into chunks of >= 4 steps until the grid holds 2048 waves
    (S <= 16 takes the tiled path only when forced, or for rows it cannot read in
    16-byte runs)."""
    with forced(WQ_FORCE_PATH="tiled"):
        kind, p = _plan(fmt, O, I, S)
    assert kind == "tiled" and int(p["ksplit"]) == ks, p
    if fmt == wq.WQ_F32:  # fp32 mode: 128 x 96 tiles from 128 rows when there are >= 128 of them
        big = S >= 128 and -(-S // 128) * -(-O // 96) >= 128
        assert (p["bm"], p["bn"], p["block"]) == (("128", "96", "256") if big else ("64", "64", "256")), p
    elif S <= 16:  # 16 x 128 tiles of eight waves side by side along o
        assert (p["bm"], p["bn"], p["block"]) == ("16", "128", "512"), p
    elif S <= 64:  # 64 x 192 tiles unless their blocks overflow a round of resident waves (int2 16384 rows)
        assert (p["bm"], p["bn"], p["block"]) == (("64", "64", "256") if O == 16384 else ("64", "192", "256")), p


def test_prefill_plan_uses_large_tiles():
    kind, p = _plan(wq.WQ_I8, 6144, 6144, 512)
    assert (p["bm"], p["bn"], p["mode"]) == ("128", "96", "bf16x3")
    assert int(p["grid"]) == 256


def _plan_gs(fmt, O, I, S, gs):
    s = wq.wq_describe_plan_gs(fmt, O, I, S, gs)
    kind, rest = s.split(" ", 1)
    return kind, dict(kv.split("=") for kv in rest.split())


@pytest.mark.parametrize("fmt,O,I,S,gs,kind", [
    (wq.WQ_I4, 12288, 6144, 2, 128, "skinny"), (wq.WQ_I4, 12288, 6144, 8, 128, "skinny"),
    (wq.WQ_I4, 12288, 6144, 12, 128, "skinny"), (wq.WQ_I2, 16384, 8192, 16, 256, "skinny"),
    (wq.WQ_I4, 12288, 6144, 16, 256, "skinny"), (wq.WQ_I8, 6144, 6144, 12, 128, "skinny"),
    (wq.WQ_I2, 16384, 8192, 8, 256, "skinny"), (wq.WQ_I4, 300, 1000, 5, 128, "skinny"),
    # a chunk would straddle two groups: int4/int8 gs % 128, int2 gs % 256
    (wq.WQ_I4, 12288, 6144, 8, 64, "tiled"), (wq.WQ_I2, 16384, 8192, 8, 128, "tiled"),
    (wq.WQ_I4, 12288, 6144, 17, 128, "tiled"),  # group scales stop at S = 16 here
    (wq.WQ_I4, 12288, 6144, 1, 128, "gemv"), (wq.WQ_I4, 12288, 6144, 8, 0, "skinny")])
def test_group_scaled_plans(fmt, O, I, S, gs, kind):
    k, p = _plan_gs(fmt, O, I, S, gs)
    assert k == kind, (k, p)
    if k == "skinny" and gs > 0:  # group-scaled tiles: two chunks in flight; 4-wave blocks for m = 3 only
        assert p["ring"] == "2" and p["waves"] in ("8", "4"), p
        if p["waves"] == "4":
            assert p["m"] == "3" and int(p["nb"]) >= 3 and int(p["grid"]) <= 256, p
    if gs == 0:
        assert wq.wq_describe_plan(fmt, O, I, S) == wq.wq_describe_plan_gs(fmt, O, I, S, 0)


def test_plan_rejects_bad_arguments():
    buf = ctypes.create_string_buffer(64)
    assert wq.lib.wq_describe_plan_gs(2, 4, 4, 1, -1, buf, 64) == wq.WQ_E_INVAL
    assert wq.lib.wq_describe_plan(9, 4, 4, 1, buf, 64) == wq.WQ_E_INVAL
    assert wq.lib.wq_describe_plan(0, 0, 4, 1, buf, 64) == wq.WQ_E_INVAL
    assert wq.lib.wq_describe_plan(0, 4, 4, -1, buf, 64) == wq.WQ_E_INVAL
    assert wq.lib.wq_describe_plan(0, 4, 4, 1, None, 64) == wq.WQ_E_INVAL


# --- argument validation happens before any HIP call -------------------------------------


def test_validation_without_device():
    L = wq.lib
    h = ctypes.c_void_p(None)
    w = np.zeros(64, np.uint8)
    sc = np.ones(4, np.float32)
    assert L.wq_tensor_upload(None, 0, 1, 4, 16, w.ctypes.data, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), 0, 9, 4, 16, w.ctypes.data, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), 0, 1, 0, 16, w.ctypes.data, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), 0, 1, 4, 0, w.ctypes.data, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), -1, 1, 4, 16, w.ctypes.data, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), 16, 1, 4, 16, w.ctypes.data, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), 0, 1, 4, 16, None, sc.ctypes.data) == wq.WQ_E_INVAL
    assert L.wq_tensor_upload(ctypes.byref(h), 0, 1, 4, 16, w.ctypes.data, None) == wq.WQ_E_INVAL
    # valid arguments, device never opened
    rc = L.wq_tensor_upload(ctypes.byref(h), 5, 1, 4, 16, w.ctypes.data, sc.ctypes.data)
    assert rc == wq.WQ_E_NOTINIT and h.value is None
    assert L.wq_matmul_t(None, None, 1, None) == wq.WQ_E_INVAL
    assert L.wq_matmul_dev(None, None, 1, None, None) == wq.WQ_E_INVAL
    assert L.wq_matmul(None, 0, 1, 4, 16, None, None, None, -1, None) == wq.WQ_E_INVAL
    assert L.wq_matmul(ctypes.byref(h), 0, 1, 4, 16, w.ctypes.data, sc.ctypes.data, None, 2, None) == wq.WQ_E_INVAL
    assert L.wq_grouped_create(None, 1, ctypes.byref(h)) == wq.WQ_E_INVAL
    assert L.wq_grouped_matmul_dev(None, None, None, None, None) == wq.WQ_E_INVAL
    assert L.wq_tensor_free(None) == wq.WQ_OK
    assert L.wq_grouped_free(None) == wq.WQ_OK
    assert L.wq_swiglu_create(None, None, 1, ctypes.byref(h)) == wq.WQ_E_INVAL
    assert L.wq_swiglu_matmul_dev(None, None, None, None, None) == wq.WQ_E_INVAL
    assert L.wq_swiglu_ffn_dev(None, None, None, None, None, None, None) == wq.WQ_E_INVAL
    assert L.wq_mem_info(-1, None, None) == wq.WQ_E_INVAL
    assert L.wq_mem_info(7, None, None) == wq.WQ_E_NOTINIT


def test_init_rejects_bad_device_lists():
    L = wq.lib
    dup = (ctypes.c_int * 2)(0, 0)
    neg = (ctypes.c_int * 1)(-1)
    big = (ctypes.c_int * 1)(16)
    many = (ctypes.c_int * 17)(*range(17))
    assert L.wq_init(dup, 2) == wq.WQ_E_INVAL
    assert L.wq_init(neg, 1) == wq.WQ_E_INVAL
    assert L.wq_init(big, 1) == wq.WQ_E_INVAL
    assert L.wq_init(many, 17) == wq.WQ_E_INVAL
    assert L.wq_init(None, 2) == wq.WQ_E_INVAL
    assert L.wq_init(None, -1) == wq.WQ_E_INVAL


def test_init_without_gpu_reports_nodev():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; the no-device path is exercised on GPU-less hosts")
    assert wq.lib.wq_init(None, 0) == wq.WQ_E_NODEV


@pytest.mark.parametrize("fmt,S,kind", [(wq.WQ_I4, 1, "gemv"), (wq.WQ_I4, 2, "skinny"), (wq.WQ_I4, 16, "skinny"),
                                        (wq.WQ_I4, 17, "skinny"), (wq.WQ_I4, 32, "skinny"), (wq.WQ_I4, 33, "tiled"),
                                        (wq.WQ_I2, 1, "gemv"), (wq.WQ_I2, 4, "skinny"), (wq.WQ_I2, 32, "skinny"),
                                        (wq.WQ_I8, 1, "gemv"), (wq.WQ_I8, 8, "skinny"), (wq.WQ_I8, 33, "tiled"),
                                        (wq.WQ_F32, 8, "gemv"), (wq.WQ_F32, 9, "tiled")])
def test_default_path_per_format_and_s(fmt, S, kind):
    """Quantized formats: the register GEMV for one activation row, the matrix-core
    few-rows kernel for 2..32, the tiled kernel above; f32 weights keep the GEMV up to
    S = 8."""
    assert _plan(fmt, 4096, 2048, S)[0] == kind


@pytest.mark.parametrize("fmt,S", [(wq.WQ_I4, 4), (wq.WQ_I2, 4), (wq.WQ_I8, 8)])
def test_unaligned_rows_keep_the_gemv(fmt, S):
    """Rows the few-rows kernel cannot read in 16-byte runs (I % 4 != 0) stay on the GEMV
    over its grouped range (S <= 4 for int4 / int2, 8 otherwise)."""
    assert _plan(fmt, 4096, 2046, S)[0] == "gemv"
    assert _plan(fmt, 4096, 2046, S + 1)[0] == "tiled"


def test_upload_gs_validation_without_device():
    """Group-scale upload: arguments are checked before any device is touched."""
    w = np.zeros((4, 64), np.uint8)   # int8 [4, 64]
    sc = np.ones((4, 1), np.float32)

    def up(fmt, gs, scales=sc, I=64):
        h = ctypes.c_void_p(None)
        return wq.lib.wq_tensor_upload_gs(ctypes.byref(h), 0, fmt, 4, I, gs, w.ctypes.data,
                                          scales.ctypes.data if scales is not None else None)
    assert up(wq.WQ_I8, 0) == wq.WQ_E_INVAL            # gs must be positive
    assert up(wq.WQ_I8, -64) == wq.WQ_E_INVAL
    assert up(wq.WQ_F32, 64) == wq.WQ_E_INVAL          # group scales are for quantized weights
    assert up(wq.WQ_I8, 32) == wq.WQ_E_UNSUPPORTED     # not a multiple of 64
    assert up(wq.WQ_I8, 100) == wq.WQ_E_UNSUPPORTED
    assert up(wq.WQ_I8, 64, scales=None) == wq.WQ_E_INVAL
    assert up(wq.WQ_I8, 64) in (wq.WQ_E_NOTINIT, wq.WQ_OK)  # valid: needs an opened device


def test_stream_read_rejects_bad_arguments_before_any_device_call():
    out = ctypes.c_void_p(0x10000)
    buf = ctypes.c_void_p(0x20000)
    f = wq.lib.wq_stream_read_dev
    assert f(None, 1024, 4, 4, out, None) == wq.WQ_E_INVAL
    assert f(buf, 1024, 4, 4, None, None) == wq.WQ_E_INVAL
    assert f(buf, 1024, 6, 4, out, None) == wq.WQ_E_INVAL      # waves not a multiple of 4
    assert f(buf, 1024, 0, 4, out, None) == wq.WQ_E_INVAL
    assert f(buf, 1024, 4, 3, out, None) == wq.WQ_E_INVAL      # uncompiled loads-in-flight count
    assert f(buf, 1000, 4, 4, out, None) == wq.WQ_E_INVAL      # not a multiple of 16 bytes
    assert f(ctypes.c_void_p(0x20008), 1024, 4, 4, out, None) == wq.WQ_E_INVAL  # misaligned
    assert f(buf, 0, 4, 4, out, None) == wq.WQ_OK              # nothing to read: no launch


@pytest.mark.parametrize("fmt,O,I,S,gs,shape", [
    (wq.WQ_I8, 6144, 6144, 512, 0, ("128", "96", "128")),   # above 64 rows: 128-deep K steps
    (wq.WQ_I2, 16384, 8192, 96, 0, ("128", "96", "128")),
    (wq.WQ_I8, 6144, 6144, 512, 128, ("128", "96", "128")),  # group scales: one group per step
    (wq.WQ_I8, 6144, 6144, 512, 192, ("128", "96", "64")),   # 192 = 1.5 steps of 128: 64-deep steps
    (wq.WQ_I4, 300, 4100, 40, 0, ("64", "64", "128")),      # 17..64 rows: 64 x 64 tiles, 128 deep
    (wq.WQ_I4, 300, 4100, 40, 64, ("64", "192", "64")),     # gs = 64: the bf16x3 rule
])
def test_bf16_activation_mode_plans(fmt, O, I, S, gs, shape):
    with forced(WQ_TILED_MODE="bf16"):
        k, p = _plan_gs(fmt, O, I, S, gs)
        assert k == "tiled" and p["mode"] == "bf16", p
        assert (p["bm"], p["bn"], p["bk"]) == shape, p
        assert int(p["workspace"]) >= int(p["tiles_s"]) * int(p["bm"]) * I * 2  # one plane
        with forced(WQ_FORCE_PATH="tiled"):  # forced at S <= 16: 64 x 64 tiles (no 16-row tile)
            k, p = _plan_gs(fmt, O, I, 9, gs)
            assert (k, p["mode"], p["bm"], p["bn"]) == ("tiled", "bf16", "64", "64"), p
    with forced(WQ_TILED_MODE="bf16x3"):
        assert _plan_gs(fmt, O, I, S, gs)[1]["mode"] == "bf16x3"


@pytest.mark.parametrize("gs,bk", [(0, "128"), (128, "128"), (256, "128"), (64, "64"), (192, "64"), (320, "64")])
def test_tiled_k_depth_follows_group_size(gs, bk):
    """128 x 96 tiles step 128 deep unless a group would straddle a step."""
    k, p = _plan_gs(wq.WQ_I8, 6144, 6144, 512, gs)
    assert (k, p["mode"], p["bm"], p["bn"], p["bk"]) == ("tiled", "bf16x3", "128", "96", bk), p
    with forced(WQ_TILED_SHAPE="128x96x128"):
        assert _plan_gs(wq.WQ_I8, 6144, 6144, 512, gs)[1]["bk"] == bk
