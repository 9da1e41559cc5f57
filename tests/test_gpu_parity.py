"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: for every output element |y_gpu - y_ref| <= 1e-5 * sum_i |scale*q*x| + 1e-30
(the oracle returns that magnitude alongside y); bit-exact where the exact
result is representable (one-hot activations, all-zero code rows, zero scales,
integer activations). Outputs are written between canary guards.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

import gpu_util as gu  # noqa: E402
import weight_only_quantized_matmul_amd as wq  # noqa: E402

F32, I8, I4, I2 = 0, 1, 2, 3


@pytest.fixture(scope="module", autouse=True)
def device():
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=None,
                       WQ_TILED_MODE=None)
    yield
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=None,
                       WQ_TILED_MODE=None)


def check_problem(p, what, x_offset=0, rows=None):
    t = gu.upload(p)
    try:
        gu.banner("%s fmt=%d O=%d I=%d S=%d plan=%s" % (what, p.fmt, p.O, p.I, p.S,
                                                        wq.wq_describe_plan(p.fmt, p.O, p.I, p.S)))
        y = gu.run_dev(t, p.x, x_offset=x_offset)
    finally:
        wq.wq_tensor_free(t)
    if rows is None:
        y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x, I=p.I)
        gu.assert_within_bound(y, y_ref, A, what)
    else:
        y_ref, A = oracle.matmul_rows(p.fmt, p.w, p.scales, p.x, rows, I=p.I)
        gu.assert_within_bound(y[:, rows], y_ref, A, what)
    return y


# ---------------------------------------------------------------------------------------
# the five workloads


@pytest.mark.parametrize("fmt", [F32, I8, I4, I2])
@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
def test_tiny_all_formats(fmt, S):
    p = synth.tiny(fmt, S=S)
    check_problem(p, "tiny")


@pytest.mark.parametrize("S", [1, 4])
def test_tiny_f32_integer_weights_and_null_scales(S):
    p = synth.tiny(F32, S=S, f32_variant="int8")
    check_problem(p, "tiny-f32-int8")
    p.scales = None
    check_problem(p, "tiny-f32-null-scales")


def test_tiny_cross_format_same_codes_identical():
    """The same int8 draw presented as f32 (exact integers) and int8 gives the same bits."""
    p8 = synth.tiny(I8, S=1)
    pf = synth.tiny(F32, S=1, f32_variant="int8")
    pf.x, pf.scales = p8.x, p8.scales
    t8, tf = gu.upload(p8), gu.upload(pf)
    try:
        y8 = gu.run_dev(t8, p8.x)
        yf = gu.run_dev(tf, pf.x)
    finally:
        wq.wq_tensor_free(t8)
        wq.wq_tensor_free(tf)
    y_ref, A = oracle.matmul(I8, p8.w, p8.scales, p8.x)
    gu.assert_within_bound(y8, y_ref, A, "i8")
    gu.assert_within_bound(yf, y_ref, A, "f32")


def test_dense_gemv_int4_full():
    check_problem(synth.dense_gemv(S=1), "dense_gemv")


@pytest.mark.parametrize("S", [1, 4, 8])
def test_int2_gemv_full(S):
    check_problem(synth.int2_gemv(S=S), "int2_gemv")


def test_prefill_int8_s512_sampled():
    p = synth.prefill(S=512)
    t = gu.upload(p)
    try:
        gu.banner("prefill plan=%s" % wq.wq_describe_plan(p.fmt, p.O, p.I, p.S))
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
    g = synth.rng(777)
    # every output row o for a sample of activation rows s (incl. the ragged last tile) ...
    s_rows = np.unique(np.concatenate([g.choice(512, 40, replace=False), [0, 63, 64, 511]]))
    y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x[s_rows])
    gu.assert_within_bound(y[s_rows], y_ref, A, "prefill rows")
    # ... and every s for a sample of output columns
    o_cols = np.unique(np.concatenate([g.choice(6144, 48, replace=False), [0, 63, 64, 6143]]))
    y_ref2, A2 = oracle.matmul_rows(p.fmt, p.w, p.scales, p.x, o_cols)
    gu.assert_within_bound(y[:, o_cols], y_ref2, A2, "prefill cols")


def test_moe_decode_grouped_one_launch():
    probs = synth.moe_decode()
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x).cuda() for p in probs]
        bufs, ys = zip(*[gu.guarded_output(p.S, p.O) for p in probs])
        gu.banner("moe grouped G=%d: launch count" % len(probs))
        # all 24 matmuls (3 KiB gate/up rows and 1 KiB down rows) in ONE kernel launch
        assert gu.count_kernel_launches(lambda: wq.wq_grouped_matmul_dev(g, xs, list(ys))) == 1
        for b in bufs:  # the capture ran nothing: reset the canaries' surroundings anyway
            b.fill_(int(np.int32(gu.CANARY.view(np.int32))))
        gu.banner("moe grouped G=%d" % len(probs))
        wq.wq_grouped_matmul_dev(g, xs, list(ys))
        torch.cuda.synchronize()
        got = []
        for p, b, y in zip(probs, bufs, ys):
            gu.check_canaries(b, p.S, p.O)
            got.append(y.cpu().numpy())
        # bit-identical to the one-tensor launches (same lane/column split and reduction order)
        for p, t, yg in zip(probs, ts, got):
            y1 = gu.run_dev(t, p.x)
            np.testing.assert_array_equal(yg, y1)
        for p, yg in zip(probs, got):
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(yg, y_ref, A, p.name)
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


def test_grouped_mixed_S_and_skips():
    probs = synth.moe_decode(n_experts=3, S=1)
    g0 = synth.rng(5)
    # give experts different activation counts, one skipped
    Ss = [3, 3, 3, 0, 0, 0, 7, 7, 7]
    for p, S in zip(probs, Ss):
        p.x = synth.activations(g0, S, p.I) if S else None
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x).cuda() if p.x is not None else None for p in probs]
        outs = [gu.guarded_output(max(p.x.shape[0], 1) if p.x is not None else 1, p.O) for p in probs]
        ys = [o[1] if p.x is not None else None for o, p in zip(outs, probs)]
        gu.banner("grouped mixed S")
        wq.wq_grouped_matmul_dev(g, xs, ys)
        torch.cuda.synchronize()
        for p, (b, y) in zip(probs, outs):
            if p.x is None:
                gu.check_canaries(b, 0, p.O)  # untouched
                continue
            gu.check_canaries(b, p.x.shape[0], p.O)
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, p.name)
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


@pytest.mark.parametrize("S", [5, 8, 16, 20, 32])
def test_grouped_few_rows_one_launch(S):
    """Several tokens per expert (above the grouped GEMV's rows): all 24
    matmuls of the 8-expert step in one launch of the few-rows kernel."""
    probs = synth.moe_decode(S=S)
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x).cuda() for p in probs]
        bufs, ys = zip(*[gu.guarded_output(p.S, p.O) for p in probs])
        gu.banner("grouped few rows S=%d: launch count" % S)
        assert gu.count_kernel_launches(lambda: wq.wq_grouped_matmul_dev(g, xs, list(ys))) == 1
        for b in bufs:
            b.fill_(int(np.int32(gu.CANARY.view(np.int32))))
        gu.banner("grouped few rows S=%d" % S)
        wq.wq_grouped_matmul_dev(g, xs, list(ys))
        torch.cuda.synchronize()
        for p, b, y in zip(probs, bufs, ys):
            gu.check_canaries(b, p.S, p.O)
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, p.name)
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt", [I8, I4, I2])
def test_grouped_few_rows_ragged_and_chunked(fmt):
    """40 tensors of ragged shapes with 0..16 rows each (some skipped): the
    few-rows kernel in launches of at most 32 active tensors."""
    g0 = synth.rng(4400 + fmt)
    probs, Ss = [], []
    for i in range(40):
        O = int(g0.integers(1, 700))
        I = 4 * int(g0.integers(1, 900))
        S = int(g0.choice([0, 1, 2, 5, 9, 13, 16]))
        S = 16 if i == 3 else S  # the launch tile is the largest S (24: four-wave blocks)
        S = 24 if (i == 5 and fmt == I8) else S
        p = synth.ragged(fmt, O, I, max(S, 1), seed=4500 + 7 * i + fmt)
        probs.append(p)
        Ss.append(S)
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x[:S]).cuda() if S else None for p, S in zip(probs, Ss)]
        outs = [gu.guarded_output(max(S, 1), p.O) for p, S in zip(probs, Ss)]
        ys = [o[1] if S else None for o, S in zip(outs, Ss)]
        active = sum(1 for S in Ss if S)
        gu.banner("grouped few rows ragged fmt=%d active=%d: launch count" % (fmt, active))
        assert gu.count_kernel_launches(lambda: wq.wq_grouped_matmul_dev(g, xs, ys)) == -(-active // 32)
        for b, _ in outs:
            b.fill_(int(np.int32(gu.CANARY.view(np.int32))))
        gu.banner("grouped few rows ragged fmt=%d" % fmt)
        wq.wq_grouped_matmul_dev(g, xs, ys)
        torch.cuda.synchronize()
        for p, S, (b, y) in zip(probs, Ss, outs):
            if S == 0:
                gu.check_canaries(b, 0, p.O)  # untouched
                continue
            gu.check_canaries(b, S, p.O)
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x[:S])
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, "%s S=%d" % (p.name, S))
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


def test_grouped_few_rows_misaligned_x_falls_back():
    """An activation buffer off a 16-byte boundary: per-tensor launches (the tiled path), same results."""
    probs = synth.moe_decode(n_experts=2, S=8)
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = []
        for p in probs:
            buf = torch.zeros(p.S * p.I + 1, dtype=torch.float32, device="cuda")
            buf[1:] = torch.from_numpy(p.x.reshape(-1)).cuda()
            xs.append(buf[1:].view(p.S, p.I))
        ys = [torch.empty((p.S, p.O), dtype=torch.float32, device="cuda") for p in probs]
        gu.banner("grouped few rows misaligned")
        wq.wq_grouped_matmul_dev(g, xs, ys)
        torch.cuda.synchronize()
        for p, y in zip(probs, ys):
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, p.name)
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt,S", [(I4, 1), (I8, 2), (I2, 1), (F32, 1)])
def test_grouped_many_problems_mixed_row_lengths(fmt, S):
    # 70 problems (two launch chunks of at most 64) whose rows need 1..4 load
    # slots: one launch per chunk, each wave on the code path of its item's
    # slot count; skipped problems in between
    g0 = synth.rng(77 + fmt + S)
    Is = [int(v) for v in g0.choice([3, 100, 700, 1500, 2100, 3000, 4000, 6000], size=70)]
    probs = []
    for j, I in enumerate(Is):
        p = synth.ragged(fmt, int(g0.integers(1, 90)), I, S, seed=4000 + j)
        if j % 9 == 4:
            p.x = None
        probs.append(p)
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x).cuda() if p.x is not None else None for p in probs]
        outs = [gu.guarded_output(S, p.O) for p in probs]
        ys = [o[1] if p.x is not None else None for o, p in zip(outs, probs)]
        gu.banner("grouped 70 problems fmt=%d S=%d" % (fmt, S))
        n = gu.count_kernel_launches(lambda: wq.wq_grouped_matmul_dev(g, xs, ys))
        if fmt == I4:  # every row fits one wave: one launch per chunk
            assert n == 2, n
        wq.wq_grouped_matmul_dev(g, xs, ys)
        torch.cuda.synchronize()
        for p, (b, y) in zip(probs, outs):
            gu.check_canaries(b, S if p.x is not None else 0, p.O)
            if p.x is None:
                continue
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, p.name)
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


# ---------------------------------------------------------------------------------------
# ragged shapes, both paths


RAGGED = [
    (F32, 1, 1, 1), (F32, 7, 13, 3), (F32, 33, 257, 9), (F32, 300, 1000, 17),
    (I8, 1, 1, 1), (I8, 5, 17, 2), (I8, 65, 1025, 8), (I8, 129, 700, 33), (I8, 200, 96, 70),
    (I4, 1, 1, 1), (I4, 3, 5, 4), (I4, 17, 33, 7), (I4, 1000, 1027, 1), (I4, 70, 2049, 12),
    (I2, 1, 3, 1), (I2, 9, 5, 2), (I2, 31, 129, 5), (I2, 600, 4097, 8), (I2, 50, 515, 65),
    (I4, 2500, 40000, 1), (I2, 100, 65000, 2), (F32, 40, 20000, 1),
]


@pytest.mark.parametrize("fmt,O,I,S", RAGGED)
def test_ragged_shapes(fmt, O, I, S):
    p = synth.ragged(fmt, O, I, S, seed=1000 + O * 7 + I * 3 + S)
    check_problem(p, "ragged")


@pytest.mark.parametrize("fmt,O,I,S", [(I4, 37, 301, 3), (I2, 20, 77, 1), (I8, 9, 43, 12), (F32, 11, 19, 2)])
def test_misaligned_activations(fmt, O, I, S):
    p = synth.ragged(fmt, O, I, S, seed=55 + O)
    check_problem(p, "misaligned-x", x_offset=1)


@pytest.mark.parametrize("path", ["gemv", "tiled", "skinny"])
@pytest.mark.parametrize("fmt,O,I,S", [(I4, 300, 776, 1), (I2, 64, 1024, 8), (I8, 128, 512, 5),
                                       (F32, 33, 100, 8), (I4, 129, 64, 2), (I8, 70, 1000, 16)])
def test_forced_paths_agree(path, fmt, O, I, S):
    p = synth.ragged(fmt, O, I, S, seed=90 + O + S)
    try:
        gu.reinit_with_env(WQ_FORCE_PATH=path)
        check_problem(p, "forced-" + path)
    finally:
        gu.reinit_with_env(WQ_FORCE_PATH=None)


# the few-rows matrix-core kernel by default (quantized, 2 <= S <= 32, I % 4 == 0):
# every (fragments, runs per lane) shape, ragged O and row tails past the permuted
# blocks, few-row plans (one 16-row block, 16 waves), the 4-wave blocks above S = 16
# with 1, 2 and 3 output blocks each, and the int4 S = 8 and S = 32 workload sizes
SKINNY_CASES = [
    (I4, 1000, 4100, 3), (I2, 777, 8196, 5), (I8, 515, 2052, 7), (I4, 2049, 1028, 9),
    (I2, 40, 4100, 12), (I8, 4097, 516, 14), (I4, 33, 12292, 6), (I2, 18, 260, 16),
    (I4, 17, 8, 2), (I8, 9000, 1028, 4), (I4, 12288, 6144, 8),
    (I4, 1000, 4100, 17), (I2, 777, 8196, 21), (I8, 515, 2052, 24), (I4, 9000, 1028, 26),
    (I2, 40, 4100, 29), (I8, 12280, 516, 32), (I4, 33, 260, 20), (I2, 13000, 2052, 18),
    (I8, 8200, 1000, 23), (I4, 12288, 6144, 32), (I8, 1, 4, 32), (I2, 5, 8, 17), (I4, 16, 4, 25),
]


@pytest.mark.parametrize("fmt,O,I,S", SKINNY_CASES)
def test_skinny_default_ragged(fmt, O, I, S):
    assert wq.wq_describe_plan(fmt, O, I, S).startswith("skinny")
    p = synth.ragged(fmt, O, I, S, seed=4242 + O + I + S)
    check_problem(p, "skinny")


@pytest.mark.parametrize("S", [8, 9, 16])
def test_gemv_tiled_crossover(S):
    p = synth.ragged(I4, 257, 1111, S, seed=31337 + S)
    check_problem(p, "crossover")


TILED_MODE_CASES = [
    (I4, 6200, 333, 130),   # 128 x 96 tiles: 2 x 65 of them, ragged in s, o and i
    (I8, 6144, 1024, 256),  # 128 x 96 tiles, exact multiples
    (I2, 300, 4100, 40),    # 64 x 64 tiles, one permuted block plus a natural tail
    (I4, 70, 2048, 9),      # 64 x 64 tiles, two permuted blocks
    (F32, 500, 999, 33),    # f32 weights always take fp32 operands
]


@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
@pytest.mark.parametrize("fmt,O,I,S", TILED_MODE_CASES)
def test_tiled_modes(mode, fmt, O, I, S):
    p = synth.ragged(fmt, O, I, S, seed=7100 + O + I + S)
    # activations over a wide exponent range exercise all three bf16 parts
    g = synth.rng(7200 + S)
    p.x = (p.x * np.exp2(g.integers(-24, 25, size=p.x.shape))).astype(np.float32)
    try:
        gu.reinit_with_env(WQ_FORCE_PATH="tiled", WQ_TILED_MODE=mode)
        plan = wq.wq_describe_plan(fmt, O, I, S)
        assert plan.startswith("tiled")
        assert ("mode=bf16x3" in plan) == (mode == "bf16x3" and fmt != F32), plan
        check_problem(p, "tiled-" + mode)
    finally:
        gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_TILED_MODE=None)


def bf16_rne(x):
    """fp32 -> the nearest bf16 (ties to even), as fp32: the rounding the
    opt-in one-plane mode applies to activations (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


@pytest.mark.parametrize("fmt,O,I,S,gs", [
    (I8, 6144, 1024, 256, 0),   # 128 x 96 tiles
    (I4, 300, 4100, 40, 0),     # 64 x 192 tiles, split K, one permuted block plus a natural tail
    (I2, 200, 1030, 70, 0),     # ragged, natural-order rows
    (I4, 500, 2048, 9, 0),      # forced tiled at S <= 16: 64 x 64 tiles (no 16-row tile in this mode)
    (I8, 257, 1000, 100, 128),  # group-wise scales, 128 x 96 tiles 128 deep
    (I4, 300, 4100, 40, 128),   # group-wise scales, 64 x 64 tiles 128 deep
    (I8, 130, 2000, 33, 0),     # 64 x 64 tiles 128 deep, split K
])
def test_tiled_bf16_activation_mode(fmt, O, I, S, gs):
    """WQ_TILED_MODE=bf16: every activation rounded to the nearest bf16, one
    plane, one MFMA per product. Pinned to the oracle on the rounded
    activations at the usual bound, and to the oracle on the fp32 activations
    within 2^-8 of the bound magnitude (the mode's contract)."""
    p = synth.ragged(fmt, O, I, S, seed=7600 + O + I + S)
    g = synth.rng(7601 + S)
    p.x = (p.x * np.exp2(g.integers(-20, 21, size=p.x.shape))).astype(np.float32)
    sc = None
    if gs:
        sc = synth.rng(7602).uniform(0.002, 0.05, size=(O, oracle.n_groups(I, gs))).astype(np.float32)
        t = wq.wq_tensor_upload_gs(None, gu.DEV, fmt, O, I, gs, p.w, sc)
    else:
        t = gu.upload(p)
    try:
        gu.reinit_with_env(WQ_FORCE_PATH="tiled", WQ_TILED_MODE="bf16")
        plan = wq.wq_describe_plan_gs(fmt, O, I, S, gs)
        assert plan.startswith("tiled") and "mode=bf16 " in plan, plan
        gu.banner("tiled bf16 activations fmt=%d O=%d I=%d S=%d gs=%d plan=%s" % (fmt, O, I, S, gs, plan))
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
        gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_TILED_MODE=None)
    xr = bf16_rne(p.x)
    if gs:
        y_r, A_r = oracle.matmul_gs(fmt, p.w, sc, gs, xr, I=I)
        y_ref, A = oracle.matmul_gs(fmt, p.w, sc, gs, p.x, I=I)
    else:
        y_r, A_r = oracle.matmul(fmt, p.w, p.scales, xr, I=I)
        y_ref, A = oracle.matmul(fmt, p.w, p.scales, p.x, I=I)
    gu.assert_within_bound(y, y_r, A_r, "bf16 mode vs rounded activations")
    err = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(err <= 2.0 ** -8 * A + 1e-30), float(np.max(err / (A + 1e-300)))
    # and the rounding is really there: the exact split's result differs
    assert np.any(y.astype(np.float64) != y_ref.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
@pytest.mark.parametrize("fmt", [I8, I4, I2])
def test_tiled_one_hot_full_mantissa(mode, fmt):
    """One nonzero activation per row, with a full 24-bit significand.

    Each output is scale * q * v rounded twice, so it is within two units in the
    last place of the exact value. Dropping any of the three bf16 parts of v
    would cost at least 2^-16 relative.
    """
    O, I, S = 40, 3000, 24
    p = synth.ragged(fmt, O, I, S, seed=7300 + fmt)
    g = synth.rng(7400 + fmt)
    cols = g.integers(0, I, size=S)
    mant = g.integers(1 << 23, 1 << 24, size=S).astype(np.float64)
    v = (mant * np.exp2(g.integers(-40, 20, size=S)) * g.choice([-1.0, 1.0], size=S)).astype(np.float32)
    x = np.zeros((S, I), np.float32)
    x[np.arange(S), cols] = v
    t = gu.upload(p)
    try:
        gu.reinit_with_env(WQ_FORCE_PATH="tiled", WQ_TILED_MODE=mode)
        gu.banner("one-hot full mantissa fmt=%d mode=%s" % (fmt, mode))
        y = gu.run_dev(t, x)
    finally:
        wq.wq_tensor_free(t)
        gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_TILED_MODE=None)
    y_ref, _ = oracle.matmul(fmt, p.w, p.scales, x)
    ref = y_ref.astype(np.float64)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= 2.0 ** -22 * np.abs(ref)), float(np.max(err / np.maximum(np.abs(ref), 1e-300)))


# ---------------------------------------------------------------------------------------
# bit-exact pins on the GPU


@pytest.mark.parametrize("fmt,I", [(I8, 256), (I4, 512), (I2, 1024)])
@pytest.mark.parametrize("S", [1, 8, 24])
def test_exhaustive_codes_one_hot_bit_exact(fmt, I, S):
    row = np.arange(256, dtype=np.uint8)[None, :]
    O = 5
    w = np.repeat(row, O, axis=0)
    sc = np.array([1.0, 0.0137, 3.5, 0.001, 123.25], dtype=np.float32)
    g = synth.rng(fmt * 10 + S)
    p = synth.Problem("exhaustive", fmt, O, I, w, sc, None)
    t = gu.upload(p)
    try:
        for c0 in range(0, I, S * 8):
            cols = np.arange(c0, min(I, c0 + S * 8), 8)[:S]
            cols = (cols + g.integers(0, 8, size=cols.size)).clip(max=I - 1)
            x = np.zeros((cols.size, I), np.float32)
            x[np.arange(cols.size), cols] = 1.0
            y = gu.run_dev(t, x)
            y_ref, _ = oracle.matmul(fmt, w, sc, x)
            np.testing.assert_array_equal(y, y_ref)
    finally:
        wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt,zero", [(I8, 0x00), (I4, 0x88), (I2, 0xAA), (F32, 0x00)])
@pytest.mark.parametrize("S", [1, 8, 40])
def test_zero_code_rows_and_zero_scales_exact(fmt, zero, S):
    p = synth.ragged(fmt, 67, 900, S, seed=4000 + fmt + S)
    p.w[5] = zero
    p.w[60] = zero
    p.scales[7] = 0.0
    p.scales[66] = 0.0
    y = check_problem(p, "zeros")
    for o in (5, 60, 7, 66):
        assert np.all(y[:, o] == 0.0), o


@pytest.mark.parametrize("fmt", [I8, I4, I2, F32])
@pytest.mark.parametrize("S", [1, 3, 8, 20])
def test_integer_activations_bit_exact(fmt, S):
    p = synth.ragged(fmt, 150, 1500, S, seed=5000 + fmt + S)
    if fmt == F32:  # f32 weights holding small integers keep every partial sum exact
        p.w = synth.f32_from_int8(synth.int8_uniform(synth.rng(5), p.O, p.I, -20, 20))
    p.x = synth.rng(6 + S).integers(-4, 5, size=(S, p.I)).astype(np.float32)
    t = gu.upload(p)
    try:
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
    y_ref, _ = oracle.matmul(fmt, p.w, p.scales, p.x)
    np.testing.assert_array_equal(y, y_ref)


def test_deterministic_repeat():
    p = synth.ragged(I4, 5000, 3000, 1, seed=99)
    t = gu.upload(p)
    try:
        y1 = gu.run_dev(t, p.x)
        y2 = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
    np.testing.assert_array_equal(y1, y2)


# ---------------------------------------------------------------------------------------
# teams of waves sharing rows, collecting row totals in LDS chunks of 32 rows

# With one wave per CU requested, each team gets many rows, so its totals
# pass through several chunks, the last one partly filled (and the last team
# ragged): int2 S=1 (two-wave teams), int4 with 10 KB rows (three-wave teams,
# 4 slots), int2 S=4 (four-wave teams, ring of 4), int8 S=8 (six-wave teams).
TEAM_CHUNK_CASES = [(I2, 5000, 8192, 1), (I4, 3001, 20000, 1), (I2, 4000, 8192, 4), (I8, 2000, 3000, 8)]


@pytest.mark.parametrize("fmt,O,I,S", TEAM_CHUNK_CASES)
def test_team_rows_over_several_chunks(fmt, O, I, S):
    gu.reinit_with_env(WQ_WAVES_PER_CU=1, WQ_FORCE_PATH="gemv")
    try:
        plan = wq.wq_describe_plan(fmt, O, I, S)
        fields = dict(kv.split("=") for kv in plan.split()[1:])
        assert plan.startswith("gemv") and int(fields["team"]) > 1 and int(fields["rows_per_team"]) > 32, plan
        p = synth.ragged(fmt, O, I, S, seed=9100 + fmt * 10 + S)
        check_problem(p, "team-chunks")
    finally:
        gu.reinit_with_env(WQ_WAVES_PER_CU=None, WQ_FORCE_PATH=None)


# ---------------------------------------------------------------------------------------
# S = 1 int4 / int2: codes enter the FMAs as exact f16 halves 2^k * q, and the
# activations meeting them are pre-divided by 2^k; activations spanning
# 1e-35 .. 1e35 stay within the bound (tiny products underflow far below its
# 1e-30 term)


@pytest.mark.parametrize("fmt,O,I", [(I4, 300, 6144), (I2, 260, 8192), (I4, 64, 1000)])
def test_s1_wide_dynamic_range_activations(fmt, O, I):
    p = synth.ragged(fmt, O, I, 1, seed=9300 + fmt)
    g = synth.rng(9301 + fmt)
    p.x = (p.x * np.power(10.0, g.uniform(-35, 35, size=p.x.shape))).astype(np.float32)
    check_problem(p, "wide-range")


@pytest.mark.parametrize("shape", ["64x64x128", "128x96x128", "64x64x64", "128x96x64"])
@pytest.mark.parametrize("fmt,O,I,S", [(I2, 300, 1030, 70), (I8, 129, 4100, 100), (I4, 1000, 2000, 40)])
def test_tiled_forced_shapes(shape, fmt, O, I, S):
    """Every compiled bf16x3 tile shape on ragged O, I and S (64- and 128-deep K steps)."""
    p = synth.ragged(fmt, O, I, S, seed=7700 + O + S)
    try:
        gu.reinit_with_env(WQ_FORCE_PATH="tiled", WQ_TILED_SHAPE=shape)
        plan = wq.wq_describe_plan(fmt, O, I, S)
        assert ("bm=%s bn=%s bk=%s" % tuple(shape.split("x"))) in plan, plan
        check_problem(p, "tiled-" + shape)
    finally:
        gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_TILED_SHAPE=None)
