"""wq_matmul_dev_noalloc (the entry point for callers that cannot allocate device
memory) through the C ABI, against wq_matmul_dev on the same inputs.

Both run the same kernels, so their outputs must agree bit for bit; each is also
held to the oracle's bound 1e-5 * sum_i |scale*q*x| + 1e-30. Two calls in a row,
the second with a smaller input, show that what the first call left in the fixed
per-device scratch array does not leak into the second. A workspace beyond the
array's size is refused before any launch.
"""
from __future__ import annotations

import ctypes

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
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=None,
                       WQ_TILED_MODE=None, WQ_TILED_SHAPE=None, WQ_WAVES_PER_CU=None)
    yield


def _noalloc_raw(t, x, y, stream):
    """The C entry point called directly (argument marshalling only)."""
    return wq.lib.wq_matmul_dev_noalloc(t.ptr, ctypes.c_void_p(x.data_ptr()), int(x.shape[0]),
                                        ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(stream.cuda_stream))


def _pair(t, p, x_rows):
    """y from wq_matmul_dev and from the no-allocation call, same inputs."""
    x = torch.from_numpy(np.ascontiguousarray(p.x[:x_rows])).cuda()
    y_dev = torch.full((x_rows, p.O), float("nan"), device="cuda")
    buf, y_na = gu.guarded_output(x_rows, p.O)
    wq.wq_matmul_dev(t, x, y_dev)
    stream = torch.cuda.current_stream()
    rc = _noalloc_raw(t, x, y_na, stream)
    assert rc == wq.WQ_OK, wq.wq_strerror(rc)
    torch.cuda.synchronize()
    gu.check_canaries(buf, x_rows, p.O)
    return y_dev.cpu().numpy(), y_na.cpu().numpy()


# (fmt, O, I, S of the first call, S of the second, smaller call): the tiled path with
# split K (workspace planes and partials), the prefill-style tile, and the register GEMV
CASES = [(I8, 2000, 3000, 40, 24), (I4, 1500, 2048, 130, 17), (I2, 1024, 4096, 12, 9), (I4, 3000, 2048, 4, 1)]


@pytest.mark.parametrize("fmt,O,I,S1,S2", CASES)
def test_noalloc_matches_matmul_dev_two_calls(fmt, O, I, S1, S2):
    p = synth.ragged(fmt, O, I, S1, seed=16000 + 10 * fmt + S1)
    t = gu.upload(p)
    try:
        for S in (S1, S2):
            plan = wq.wq_describe_plan(fmt, O, I, S)
            gu.banner("noalloc fmt=%d O=%d I=%d S=%d plan=%s" % (fmt, O, I, S, plan))
            y_dev, y_na = _pair(t, p, S)
            np.testing.assert_array_equal(y_na, y_dev)
            y_ref, A = oracle.matmul(fmt, p.w, p.scales, p.x[:S])
            gu.assert_within_bound(y_na, y_ref, A, "noalloc S=%d" % S)
    finally:
        wq.wq_tensor_free(t)


def test_noalloc_refuses_workspace_beyond_its_array():
    O, I, S = 64, 8192, 2048  # planes alone: 3 * 2048 * 8192 * 2 bytes = 96 MiB
    assert wq.wq_noalloc_scratch_bytes() == 32 << 20
    plan = wq.wq_describe_plan(I8, O, I, S)
    assert int(plan.split("workspace=")[1]) > wq.wq_noalloc_scratch_bytes(), plan
    p = synth.ragged(I8, O, I, 1, seed=16100)
    t = gu.upload(p)
    try:
        x = torch.zeros((S, I), device="cuda")
        y = torch.full((S, O), 7.0, device="cuda")
        rc = _noalloc_raw(t, x, y, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert rc == wq.WQ_E_UNSUPPORTED
        assert torch.all(y == 7.0)  # nothing was launched
    finally:
        wq.wq_tensor_free(t)


def test_noalloc_in_a_captured_graph_replays_like_eager():
    """The use it exists for: captured without any warm-up (no workspace to grow)."""
    p = synth.ragged(I8, 1000, 1500, 100, seed=16200)
    t = gu.upload(p)
    try:
        x = torch.from_numpy(p.x).cuda()
        y_graph = torch.zeros((p.S, p.O), device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        gu.banner("noalloc capture: %s" % wq.wq_describe_plan(I8, p.O, p.I, p.S))
        with torch.cuda.graph(g, stream=side):
            wq.wq_matmul_dev_noalloc(t, x, y_graph)
        torch.cuda.synchronize()
        y_ref, A = oracle.matmul(I8, p.w, p.scales, p.x)
        y_eager = None
        for i in range(3):
            y_graph.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = y_graph.cpu().numpy()
            gu.assert_within_bound(got, y_ref, A, "noalloc replay %d" % i)
            if y_eager is None:
                ye = torch.empty_like(y_graph)
                wq.wq_matmul_dev(t, x, ye)
                torch.cuda.synchronize()
                y_eager = ye.cpu().numpy()
            np.testing.assert_array_equal(got, y_eager)
            # eager work between replays, writing the same scratch array
            yo = torch.empty_like(y_graph)
            wq.wq_matmul_dev_noalloc(t, x[:37], yo[:37])
            torch.cuda.synchronize()
    finally:
        wq.wq_tensor_free(t)
