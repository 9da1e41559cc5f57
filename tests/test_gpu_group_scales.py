"""GPU parity for tensors with group-wise scales (one scale per output row and
group of gs columns) against the oracle's matmul_gs, through the C ABI."""
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

I8, I4, I2 = 1, 2, 3


@pytest.fixture(scope="module", autouse=True)
def device():
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_TILED_MODE=None, WQ_TILED_SHAPE=None)
    yield


def gscales(seed, O, I, gs, lo=0.002, hi=0.05):
    return synth.rng(seed).uniform(lo, hi, size=(O, oracle.n_groups(I, gs))).astype(np.float32)


def upload_gs(fmt, O, I, gs, w, sc):
    return wq.wq_tensor_upload_gs(None, gu.DEV, fmt, O, I, gs, w, sc)


def check(fmt, O, I, S, gs, seed, rows=None, what="gs", x_offset=0):
    p = synth.ragged(fmt, O, I, S, seed=seed)
    sc = gscales(seed + 1, O, I, gs)
    t = upload_gs(fmt, O, I, gs, p.w, sc)
    try:
        gu.banner("%s fmt=%d O=%d I=%d S=%d gs=%d x_offset=%d plan=%s" % (what, fmt, O, I, S, gs, x_offset,
                                                                         wq.wq_describe_plan_gs(fmt, O, I, S, gs)))
        y = gu.run_dev(t, p.x, x_offset=x_offset)
    finally:
        wq.wq_tensor_free(t)
    if rows is None:
        y_ref, A = oracle.matmul_gs(fmt, p.w, sc, gs, p.x)
        gu.assert_within_bound(y, y_ref, A, what)
    else:
        y_ref, A = oracle.matmul_gs_rows(fmt, p.w, sc, gs, p.x, rows)
        gu.assert_within_bound(y[:, rows], y_ref, A, what)
    return y


@pytest.mark.parametrize("fmt", [I8, I4, I2])
@pytest.mark.parametrize("gs", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 20, 130])
def test_group_scales_parity(fmt, gs, S):
    check(fmt, 300, 1000, S, gs, seed=8000 + 100 * fmt + gs + S)


@pytest.mark.parametrize("fmt,O,I,S,gs", [(I4, 129, 64, 1, 64), (I2, 70, 4100, 2, 1024), (I8, 33, 5000, 9, 64),
                                         (I4, 1000, 3000, 4, 4096), (I2, 17, 130, 40, 128),
                                         # S = 1 rows of 2, 3 and 4 load slots per lane, and a team of
                                         # several waves per row (int8 20000 bytes, int2 9000 elements)
                                         (I8, 77, 2500, 1, 64), (I4, 91, 7000, 1, 128), (I4, 60, 8192, 1, 256),
                                         (I8, 50, 20000, 1, 128), (I2, 45, 9000, 1, 64)])
def test_group_scales_ragged(fmt, O, I, S, gs):
    check(fmt, O, I, S, gs, seed=8500 + O + I + S, what="gs-ragged")


@pytest.mark.parametrize("fmt,O,I,gs", [(I4, 70, 6144, 128), (I4, 33, 8192, 64), (I8, 40, 3000, 128),
                                       (I2, 50, 8192, 256)])
def test_group_scales_misaligned_activations(fmt, O, I, gs):
    """S = 1 with x one float past a 16-byte boundary: the GEMV reads it element by element."""
    check(fmt, O, I, 1, gs, seed=8550 + O + I, what="gs-misaligned", x_offset=1)


@pytest.mark.parametrize("shape", ["64x192x64", "64x64x64", "128x96x64", "128x96x128", "64x64x128"])
@pytest.mark.parametrize("fmt,O,I,S,gs", [(I4, 500, 3000, 40, 128), (I8, 200, 1000, 20, 64), (I2, 300, 4100, 50, 256)])
def test_group_scales_forced_tile_shapes(shape, fmt, O, I, S, gs):
    """Every group-scaled tiled kernel (the group sums added per K step; a 128-deep
    shape with gs = 64 plans 64-deep steps instead)."""
    try:
        gu.reinit_with_env(WQ_FORCE_PATH="tiled", WQ_TILED_SHAPE=shape)
        check(fmt, O, I, S, gs, seed=8900 + O + S, what="gs-tile-" + shape)
    finally:
        gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_TILED_SHAPE=None)


# Few activation rows on the matrix cores with group scales: ragged o blocks
# (O not a multiple of 16 * nb), ragged last chunk and group, every compiled
# stack of fragments (S = 2..16) and several groups per chunk pair (gs = 128)
# or chunks per group (gs >= 256).
@pytest.mark.parametrize("fmt,O,I,S,gs", [(I4, 300, 1000, 2, 128), (I4, 517, 3000, 5, 384), (I4, 70, 2048, 6, 128),
                                         (I4, 1000, 6144, 11, 256), (I4, 45, 1100, 16, 128),
                                         (I8, 300, 1000, 4, 128), (I8, 257, 2500, 9, 256), (I8, 129, 640, 13, 128),
                                         (I2, 300, 1000, 3, 256), (I2, 700, 4100, 8, 512), (I2, 60, 8192, 16, 256),
                                         # many output rows at 11..16 rows: 4-wave blocks of 3-4 output blocks
                                         (I8, 9000, 700, 14, 128), (I4, 10000, 1300, 16, 256),
                                         (I2, 12000, 1032, 12, 256)])
def test_group_scales_few_rows_kernel(fmt, O, I, S, gs):
    assert wq.wq_describe_plan_gs(fmt, O, I, S, gs).startswith("skinny")
    check(fmt, O, I, S, gs, seed=8700 + O + I + S + gs, what="gs-skinny")


@pytest.mark.parametrize("S", [2, 8, 16])
def test_group_scales_few_rows_decode_shape(S):
    """int4 12288 x 6144, gs = 128, the batched-decode shapes, on sampled rows."""
    assert wq.wq_describe_plan_gs(I4, 12288, 6144, S, 128).startswith("skinny")
    rows = np.arange(5, 12288, 89)
    check(I4, 12288, 6144, S, 128, seed=8650 + S, rows=rows, what="gs-skinny-dense")


def test_group_scales_few_rows_bit_identical_to_forced_tiled_on_integers():
    """Integer activations and integer group scales: every partial sum is an
    exact integer below 2^24, so the few-rows kernel and the tiled kernel must
    agree bit for bit (and with the oracle)."""
    fmt, O, I, S, gs = I4, 200, 1024, 8, 128
    p = synth.ragged(fmt, O, I, S, seed=8800)
    p.x = synth.rng(8801).integers(-4, 5, size=(S, I)).astype(np.float32)
    sc = synth.rng(8802).integers(1, 4, size=(O, oracle.n_groups(I, gs))).astype(np.float32)
    t = upload_gs(fmt, O, I, gs, p.w, sc)
    try:
        assert wq.wq_describe_plan_gs(fmt, O, I, S, gs).startswith("skinny")
        gu.banner("gs integers skinny")
        y1 = gu.run_dev(t, p.x)
        gu.reinit_with_env(WQ_FORCE_PATH="tiled")
        gu.banner("gs integers tiled")
        y2 = gu.run_dev(t, p.x)
    finally:
        gu.reinit_with_env(WQ_FORCE_PATH=None)
        wq.wq_tensor_free(t)
    y_ref, _ = oracle.matmul_gs(fmt, p.w, sc, gs, p.x)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(y1, y_ref.astype(np.float32))


def test_group_scales_dense_decode_shape():
    rows = np.arange(0, 12288, 97)
    check(I4, 12288, 6144, 1, 128, seed=8600, rows=rows, what="gs-dense")


def test_group_scales_prefill_shape():
    rows = np.arange(0, 6144, 191)
    check(I8, 6144, 6144, 512, 128, seed=8601, rows=rows, what="gs-prefill")


@pytest.mark.parametrize("fmt,I", [(I8, 256), (I4, 512), (I2, 1024)])
@pytest.mark.parametrize("S", [1, 8, 24])
def test_group_scales_one_hot_bit_exact(fmt, I, S):
    gs = 64
    row = np.arange(256, dtype=np.uint8)[None, :]
    O = 4
    w = np.repeat(row, O, axis=0)
    sc = gscales(8700 + fmt, O, I, gs, 0.01, 3.0)
    t = upload_gs(fmt, O, I, gs, w, sc)
    g = synth.rng(8710 + fmt + S)
    try:
        for c0 in range(0, I, S * 8):
            cols = np.arange(c0, min(I, c0 + S * 8), 8)[:S]
            cols = (cols + g.integers(0, 8, size=cols.size)).clip(max=I - 1)
            x = np.zeros((cols.size, I), np.float32)
            x[np.arange(cols.size), cols] = 1.0
            gu.banner("gs one-hot fmt=%d S=%d c0=%d" % (fmt, x.shape[0], c0))
            y = gu.run_dev(t, x)
            y_ref, _ = oracle.matmul_gs(fmt, w, sc, gs, x)
            np.testing.assert_array_equal(y, y_ref)
    finally:
        wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt,zero", [(I8, 0x00), (I4, 0x88), (I2, 0xAA)])
@pytest.mark.parametrize("S", [1, 8, 40])
def test_group_scales_zero_rows_exact(fmt, zero, S):
    O, I, gs = 67, 900, 128
    p = synth.ragged(fmt, O, I, S, seed=8800 + fmt + S)
    sc = gscales(8801 + fmt, O, I, gs)
    p.w[5] = zero          # all codes decode to 0
    sc[7] = 0.0            # every group scale of a row is 0
    sc[20, 1] = 0.0        # one group of a row is 0: only that group drops out
    t = upload_gs(fmt, O, I, gs, p.w, sc)
    try:
        gu.banner("gs zeros fmt=%d S=%d" % (fmt, S))
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
    assert np.all(y[:, 5] == 0.0) and np.all(y[:, 7] == 0.0)
    y_ref, A = oracle.matmul_gs(fmt, p.w, sc, gs, p.x)
    gu.assert_within_bound(y, y_ref, A, "gs zeros")


@pytest.mark.parametrize("S", [1, 2, 8, 16])
def test_group_scales_in_a_group_call(S):
    """Grouped calls holding group-scaled tensors: per tensor at S = 1, one
    few-rows launch for 2..16 rows."""
    probs = [synth.ragged(I4, 512, 2048, S, seed=8900 + k + S) for k in range(3)]
    scs = [gscales(8950 + k, 512, 2048, 128) for k in range(3)]
    ts = [upload_gs(I4, 512, 2048, 128, p.w, sc) for p, sc in zip(probs, scs)]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x).cuda() for p in probs]
        ys = [torch.empty((S, 512), device="cuda") for _ in probs]
        if S > 1:
            wq.wq_grouped_matmul_dev(g, xs, ys)
            torch.cuda.synchronize()
            gu.banner("gs grouped call S=%d: launch count" % S)
            assert gu.count_kernel_launches(lambda: wq.wq_grouped_matmul_dev(g, xs, ys)) == 1
        gu.banner("gs grouped call S=%d" % S)
        wq.wq_grouped_matmul_dev(g, xs, ys)
        torch.cuda.synchronize()
        for p, sc, y in zip(probs, scs, ys):
            y_ref, A = oracle.matmul_gs(I4, p.w, sc, 128, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, "gs grouped")
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt,gs", [(I8, 256), (I4, 128), (I2, 256)])
def test_group_scales_mixed_group_few_rows(fmt, gs):
    """A group mixing group-scaled tensors (gs) and tensors with one scale per
    row, 2..16 rows each, some skipped: one group-scaled few-rows launch (a
    row-scaled tensor is one group as long as its row)."""
    g0 = synth.rng(8960 + fmt)
    probs, scs, Ss = [], [], []
    for k in range(7):
        O, I = int(g0.integers(20, 600)), 4 * int(g0.integers(40, 700))
        S = [3, 0, 16, 8, 2, 5, 11][k]
        p = synth.ragged(fmt, O, I, max(S, 1), seed=8970 + k + fmt)
        probs.append(p)
        scs.append(gscales(8990 + k, O, I, gs) if k % 2 == 0 else None)
        Ss.append(S)
    ts = [upload_gs(fmt, p.O, p.I, gs, p.w, sc) if sc is not None else gu.upload(p) for p, sc in zip(probs, scs)]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x[:S]).cuda() if S else None for p, S in zip(probs, Ss)]
        ys = [torch.empty((S, p.O), device="cuda") if S else None for p, S in zip(probs, Ss)]
        gu.banner("gs mixed group few rows fmt=%d: launch count" % fmt)
        assert gu.count_kernel_launches(lambda: wq.wq_grouped_matmul_dev(g, xs, ys)) == 1
        gu.banner("gs mixed group few rows fmt=%d" % fmt)
        wq.wq_grouped_matmul_dev(g, xs, ys)
        torch.cuda.synchronize()
        for p, sc, S, y in zip(probs, scs, Ss, ys):
            if S == 0:
                continue
            if sc is None:
                y_ref, A = oracle.matmul(fmt, p.w, p.scales, p.x[:S])
            else:
                y_ref, A = oracle.matmul_gs(fmt, p.w, sc, gs, p.x[:S])
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, "gs mixed group")
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


def test_group_scale_reupload_checks_gs():
    p = synth.ragged(I8, 16, 256, 1, seed=9000)
    sc = gscales(9001, 16, 256, 64)
    t = upload_gs(I8, 16, 256, 64, p.w, sc)
    try:
        assert wq.wq_tensor_upload_gs(t, gu.DEV, I8, 16, 256, 64, None, None) is t
        with pytest.raises(wq.WqError) as ei:
            wq.wq_tensor_upload_gs(t, gu.DEV, I8, 16, 256, 128, None, None)
        assert ei.value.code == wq.WQ_E_MISMATCH
        with pytest.raises(wq.WqError) as ei:
            wq.wq_tensor_upload(t, gu.DEV, I8, 16, 256, None, None)
        assert ei.value.code == wq.WQ_E_MISMATCH
    finally:
        wq.wq_tensor_free(t)


def test_group_scales_split_team_over_several_chunks():
    """Group-scaled rows are split over one-slot teams; with one wave per CU
    requested each team's totals pass through several 32-row LDS chunks."""
    gu.reinit_with_env(WQ_WAVES_PER_CU=1)
    try:
        check(I4, 3000, 6144, 1, 128, seed=9500, what="gs-team-chunks")
        check(I2, 2100, 8192, 2, 256, seed=9510, what="gs-team-chunks")
    finally:
        gu.reinit_with_env(WQ_WAVES_PER_CU=None)
