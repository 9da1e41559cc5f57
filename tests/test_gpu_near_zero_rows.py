"""GPU parity on near-zero rows: rows whose codes all sit at the zero point
(int4 nibble 8, int2 code 2) except one to three fields.

The contract bounds the error of every output element by
1e-5 * sum_i |scale*q*x| + 1e-30. On such rows that magnitude comes from the
few non-zero fields alone, so a kernel whose rounding scales with anything
larger -- for instance with sum_i |code*x| when the offset is subtracted as
offset * sum(x) after the sum -- fails here, most of all when the non-zero
fields meet the smallest activations. Dequantization rule: colibri-analysis
"CUDA 后端", section 1 (weight_at: int4 minus 8, int2 minus 2).

Covered paths: the single-tensor call (S = 1, 2, 4, and a tiled S), the
grouped launch, the gated (SwiGLU) launch and group-wise scales.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import packing
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)

import gpu_util as gu  # noqa: E402
import weight_only_quantized_matmul_amd as wq  # noqa: E402

I8, I4, I2 = 1, 2, 3
QRANGE = {I8: (-127, 127), I4: (-8, 7), I2: (-2, 1)}


@pytest.fixture(scope="module", autouse=True)
def device():
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=None,
                       WQ_TILED_MODE=None, WQ_TILED_SHAPE=None, WQ_WAVES_PER_CU=None)
    yield


def near_zero_problem(fmt, O, I, S, seed, smallest=False, kmax=3):
    """Packed weights with every value 0 except 1..kmax fields per row (non-zero values,
    uniform over the format's range); with smallest=True those fields sit on the columns
    of the smallest |x[0, i]|."""
    g = synth.rng(seed)
    x = synth.activations(g, S, I)
    vals = np.zeros((O, I), dtype=np.int64)
    lo, hi = QRANGE[fmt]
    pool = np.argsort(np.abs(x[0]), kind="stable")[:64] if smallest else None
    for o in range(O):
        k = int(g.integers(1, kmax + 1))
        cols = g.choice(pool, size=k, replace=False) if smallest else g.choice(I, size=k, replace=False)
        v = g.integers(lo, hi, size=k)  # lo .. hi-1, then skip 0
        v[v >= 0] += 1
        vals[o, cols] = v
    w = packing.pack(fmt, vals)
    sc = synth.scales(g, O, 0.002, 0.05)
    return synth.Problem("near_zero_%d" % fmt, fmt, O, I, w, sc, x)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:%d" % gu.DEV)


CASES = [(I4, 256, 6144), (I2, 256, 8192), (I4, 300, 1000), (I8, 128, 6144)]


@pytest.mark.parametrize("fmt,O,I", CASES)
@pytest.mark.parametrize("S", [1, 2, 4, 24])
@pytest.mark.parametrize("smallest", [False, True])
def test_near_zero_rows_single(fmt, O, I, S, smallest):
    p = near_zero_problem(fmt, O, I, S, seed=12000 + 10 * fmt + S + (5 if smallest else 0), smallest=smallest)
    t = gu.upload(p)
    try:
        gu.banner("near-zero fmt=%d O=%d I=%d S=%d smallest=%s plan=%s" % (
            fmt, O, I, S, smallest, wq.wq_describe_plan(fmt, O, I, S)))
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
    y_ref, A = oracle.matmul(fmt, p.w, p.scales, p.x)
    gu.assert_within_bound(y, y_ref, A, "near-zero single")


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("smallest", [False, True])
def test_near_zero_rows_grouped(S, smallest):
    # the moe_decode shapes at reduced O: 3 KiB gate/up rows and 1 KiB down rows
    probs = []
    for e in range(2):
        base = 13000 + 100 * e + S + (50 if smallest else 0)
        probs += [near_zero_problem(I4, 256, 6144, S, base, smallest),
                  near_zero_problem(I4, 256, 6144, S, base + 1, smallest),
                  near_zero_problem(I4, 384, 2048, S, base + 2, smallest)]
    ts = [gu.upload(p) for p in probs]
    grp = wq.wq_grouped_create(ts)
    try:
        xs = [dev(p.x) for p in probs]
        bufs = [gu.guarded_output(p.S, p.O) for p in probs]
        gu.banner("near-zero grouped S=%d smallest=%s" % (S, smallest))
        wq.wq_grouped_matmul_dev(grp, xs, [b[1] for b in bufs])
        torch.cuda.synchronize()
        for p, (buf, y) in zip(probs, bufs):
            gu.check_canaries(buf, p.S, p.O)
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, "near-zero grouped")
    finally:
        wq.wq_grouped_free(grp)
        for t in ts:
            wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt,I", [(I4, 6144), (I2, 8192)])
@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("smallest", [False, True])
def test_near_zero_rows_swiglu(fmt, I, S, smallest):
    base = 14000 + 10 * fmt + S + (5 if smallest else 0)
    gates = [near_zero_problem(fmt, 192, I, S, base + 2 * e, smallest) for e in range(2)]
    ups = [near_zero_problem(fmt, 192, I, S, base + 2 * e + 1, smallest) for e in range(2)]
    for gp, up in zip(gates, ups):
        up.x = gp.x  # gate and up read the same activations
    gts = [gu.upload(p) for p in gates]
    uts = [gu.upload(p) for p in ups]
    grp = wq.wq_swiglu_create(gts, uts)
    try:
        xs = [dev(p.x) for p in gates]
        bufs = [gu.guarded_output(p.S, p.O) for p in gates]
        gu.banner("near-zero swiglu fmt=%d S=%d smallest=%s" % (fmt, S, smallest))
        wq.wq_swiglu_matmul_dev(grp, xs, [b[1] for b in bufs])
        torch.cuda.synchronize()
        for gp, up, (buf, h) in zip(gates, ups, bufs):
            gu.check_canaries(buf, gp.S, gp.O)
            gv, ag = oracle.matmul(fmt, gp.w, gp.scales, gp.x)
            uv, au = oracle.matmul(fmt, up.w, up.scales, gp.x)
            ref = {"g": gv, "Ag": ag, "u": uv, "Au": au, "h": oracle.silu_mul(gv, uv)}
            gu.assert_h(h.cpu().numpy(), ref, "near-zero swiglu")
    finally:
        wq.wq_grouped_free(grp)
        for t in gts + uts:
            wq.wq_tensor_free(t)


@pytest.mark.parametrize("fmt,I,gs", [(I4, 6144, 128), (I2, 8192, 128), (I2, 8192, 256)])
@pytest.mark.parametrize("S", [1, 2, 8, 24])
def test_near_zero_rows_group_scales(fmt, I, gs, S):
    p = near_zero_problem(fmt, 200, I, S, seed=15000 + 10 * fmt + S, smallest=True)
    gsc = synth.rng(15001 + S).uniform(0.002, 0.05, size=(p.O, oracle.n_groups(I, gs))).astype(np.float32)
    t = wq.wq_tensor_upload_gs(None, gu.DEV, fmt, p.O, I, gs, p.w, gsc)
    try:
        gu.banner("near-zero gs=%d fmt=%d S=%d plan=%s" % (gs, fmt, S, wq.wq_describe_plan_gs(fmt, p.O, I, S, gs)))
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
    y_ref, A = oracle.matmul_gs(fmt, p.w, gsc, gs, p.x)
    gu.assert_within_bound(y, y_ref, A, "near-zero group scales")
