"""GPU tests of the C ABI around the kernels: host-pointer calls, lazy upload,
re-upload validation, memory info, injected failures, graph capture."""
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


@pytest.fixture(autouse=True)
def device():
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=None, WQ_TILED_SHAPE=None,
                       WQ_TILED_MODE=None)
    yield
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=None, WQ_TILED_SHAPE=None,
                       WQ_TILED_MODE=None)


def test_mem_info():
    free, total = wq.wq_mem_info(0)
    assert 0 < free <= total
    assert total > 200 * 2**30  # MI355X carries 288 GB of HBM3E


def test_lazy_matmul_uploads_once_and_matches_oracle():
    p = synth.ragged(I4, 500, 1000, 3, seed=11)
    gu.banner("wq_matmul lazy")
    t, y = wq.wq_matmul(None, 0, p.fmt, p.O, p.I, p.w, p.scales, p.x)
    try:
        y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
        gu.assert_within_bound(y, y_ref, A, "wq_matmul")
        # second call with the handle: no upload; garbage weights are not even read
        t2, y2 = wq.wq_matmul(t, 0, p.fmt, p.O, p.I, None, None, p.x)
        assert t2 is t
        np.testing.assert_array_equal(y, y2)
        y3 = wq.wq_matmul_t(t, p.x)
        np.testing.assert_array_equal(y, y3)
        # the device-pointer path gives the same bits
        np.testing.assert_array_equal(gu.run_dev(t, p.x), y)
    finally:
        wq.wq_tensor_free(t)


def test_reupload_validates_only():
    p = synth.ragged(I8, 10, 20, 1, seed=12)
    t = wq.wq_tensor_upload(None, 0, p.fmt, p.O, p.I, p.w, p.scales)
    try:
        assert wq.wq_tensor_upload(t, 0, p.fmt, p.O, p.I, None, None) is t
        for bad in [(0, I4, p.O, p.I), (0, p.fmt, p.O + 1, p.I), (0, p.fmt, p.O, p.I + 1)]:
            with pytest.raises(wq.WqError) as e:
                wq.wq_tensor_upload(t, *bad, None, None)
            assert e.value.code == wq.WQ_E_MISMATCH
    finally:
        wq.wq_tensor_free(t)


def test_s_zero_is_a_noop():
    p = synth.ragged(I2, 10, 20, 1, seed=13)
    t = gu.upload(p)
    try:
        x = np.zeros((0, p.I), np.float32)
        assert wq.wq_matmul_t(t, x).shape == (0, p.O)
        assert wq.lib.wq_matmul_dev(t.ptr, None, 0, None, None) == wq.WQ_OK
    finally:
        wq.wq_tensor_free(t)


def test_host_call_large_then_small_reuses_scratch():
    big = synth.ragged(I4, 3000, 4000, 8, seed=14)
    small = synth.ragged(I4, 3000, 4000, 1, seed=15)
    small.w, small.scales = big.w, big.scales
    t = gu.upload(big)
    try:
        for p in (big, small, big):
            y = wq.wq_matmul_t(t, p.x)
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y, y_ref, A, "host S=%d" % p.S)
    finally:
        wq.wq_tensor_free(t)


def test_injected_launch_failure_leaves_output_untouched():
    p = synth.ragged(I4, 64, 128, 2, seed=16)
    t = gu.upload(p)
    try:
        gu.reinit_with_env(WQ_FAULT="launch")
        xd = torch.from_numpy(p.x).cuda()
        buf, y = gu.guarded_output(p.S, p.O)
        with pytest.raises(wq.WqError) as e:
            wq.wq_matmul_dev(t, xd, y)
        assert e.value.code == wq.WQ_E_FAULT
        torch.cuda.synchronize()
        gu.check_canaries(buf, 0, p.O)  # nothing written at all
        with pytest.raises(wq.WqError):
            wq.wq_matmul_t(t, p.x)
    finally:
        gu.reinit_with_env(WQ_FAULT=None)
        wq.wq_tensor_free(t)


def test_injected_upload_failure_and_memory_budget():
    p = synth.ragged(I4, 64, 128, 1, seed=17)
    gu.reinit_with_env(WQ_FAULT="upload")
    with pytest.raises(wq.WqError) as e:
        gu.upload(p)
    assert e.value.code == wq.WQ_E_FAULT
    gu.reinit_with_env(WQ_FAULT=None, WQ_MEM_LIMIT_BYTES=1000)
    with pytest.raises(wq.WqError) as e:
        gu.upload(p)  # 64*64 + 256 bytes > 1000
    assert e.value.code == wq.WQ_E_OOM
    gu.reinit_with_env(WQ_MEM_LIMIT_BYTES=None)
    t = gu.upload(p)
    wq.wq_tensor_free(t)


def test_grouped_rejects_mixed_formats():
    a = gu.upload(synth.ragged(I4, 8, 16, 1, seed=18))
    b = gu.upload(synth.ragged(I8, 8, 16, 1, seed=19))
    try:
        with pytest.raises(wq.WqError) as e:
            wq.wq_grouped_create([a, b])
        assert e.value.code == wq.WQ_E_INVAL
    finally:
        wq.wq_tensor_free(a)
        wq.wq_tensor_free(b)


def test_graph_capture_replays_match_eager():
    p = synth.ragged(I4, 4096, 2048, 1, seed=20)
    t = gu.upload(p)
    try:
        x = torch.from_numpy(p.x).cuda()
        y_eager = torch.empty((p.S, p.O), device="cuda")
        wq.wq_matmul_dev(t, x, y_eager)
        torch.cuda.synchronize()
        y_graph = torch.zeros_like(y_eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            wq.wq_matmul_dev(t, x, y_graph)
        torch.cuda.synchronize()
        for i in range(4):
            y_graph.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_graph, y_eager), "replay %d differs" % i
            wq.wq_matmul_dev(t, x, y_eager)  # eager work between replays
            torch.cuda.synchronize()
    finally:
        wq.wq_tensor_free(t)


def test_grouped_call_capture_mixed_row_lengths():
    """A grouped call over rows of two slot counts (gate/up rows and down rows,
    one launch), captured in a graph and replayed, matches eager."""
    probs = synth.moe_decode(n_experts=3, S=1)
    ts = [gu.upload(p) for p in probs]
    g = wq.wq_grouped_create(ts)
    try:
        xs = [torch.from_numpy(p.x).cuda() for p in probs]
        ys_eager = [torch.empty((p.S, p.O), device="cuda") for p in probs]
        ys_graph = [torch.zeros_like(y) for y in ys_eager]
        gu.banner("grouped capture, mixed row lengths")
        wq.wq_grouped_matmul_dev(g, xs, ys_eager)
        torch.cuda.synchronize()
        for p, y in zip(probs, ys_eager):
            y_ref, A = oracle.matmul(p.fmt, p.w, p.scales, p.x)
            gu.assert_within_bound(y.cpu().numpy(), y_ref, A, p.name)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            wq.wq_grouped_matmul_dev(g, xs, ys_graph)
        torch.cuda.synchronize()
        for i in range(4):
            for y in ys_graph:
                y.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for y, ye in zip(ys_graph, ys_eager):
                assert torch.equal(y, ye), "replay %d differs" % i
            wq.wq_grouped_matmul_dev(g, xs, ys_eager)  # eager work between replays
            torch.cuda.synchronize()
    finally:
        wq.wq_grouped_free(g)
        for t in ts:
            wq.wq_tensor_free(t)


def _capture(t, x, y):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        wq.wq_matmul_dev(t, x, y)
    torch.cuda.synchronize()
    return g


def test_graph_capture_tiled_after_warmup():
    """The tiled path (split pre-pass + MFMA kernel, device workspace) replays like eager."""
    p = synth.ragged(I8, 1000, 1500, 100, seed=21)
    t = gu.upload(p)
    try:
        x = torch.from_numpy(p.x).cuda()
        y_eager = torch.empty((p.S, p.O), device="cuda")
        gu.banner("capture tiled warmup: %s" % wq.wq_describe_plan(I8, p.O, p.I, p.S))
        wq.wq_matmul_dev(t, x, y_eager)  # sizes the workspace outside the capture
        torch.cuda.synchronize()
        y_ref, A = oracle.matmul(I8, p.w, p.scales, p.x)
        gu.assert_within_bound(y_eager.cpu().numpy(), y_ref, A, "eager tiled")
        y_graph = torch.zeros_like(y_eager)
        g = _capture(t, x, y_graph)
        for i in range(4):
            y_graph.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_graph, y_eager), "replay %d differs" % i
            wq.wq_matmul_dev(t, x, y_eager)  # eager work between replays
            torch.cuda.synchronize()
    finally:
        wq.wq_tensor_free(t)


def test_capture_refuses_workspace_growth():
    """A captured call never allocates: a larger S than any eager call so far is refused."""
    p = synth.ragged(I4, 300, 20000, 4000, seed=22)  # more workspace than every other test uses
    t = gu.upload(p)
    try:
        plan = wq.wq_describe_plan(I4, p.O, p.I, p.S)
        assert "mode=bf16x3" in plan, plan
        x = torch.from_numpy(p.x).cuda()
        y = torch.zeros((p.S, p.O), device="cuda")
        gu.banner("capture refused: " + plan)
        with pytest.raises(wq.WqError) as ei:
            _capture(t, x, y)
        assert ei.value.code == wq.WQ_E_UNSUPPORTED
        torch.cuda.synchronize()
        # the same call eagerly grows the workspace and is correct
        wq.wq_matmul_dev(t, x, y)
        torch.cuda.synchronize()
        rows = np.arange(0, p.O, 37)
        yh = y.cpu().numpy()
        y_ref, A = oracle.matmul_rows(I4, p.w, p.scales, p.x, rows)
        gu.assert_within_bound(yh[:, rows], y_ref, A, "after growth")
    finally:
        wq.wq_tensor_free(t)


def _tiled_case(seed):
    """An int8 tensor on the tiled path and two activation sets of different S (both tiled)."""
    p = synth.ragged(I8, 1536, 4096, 256, seed=seed)
    rng = np.random.default_rng(seed + 1)
    x2 = rng.standard_normal((200, p.I)).astype(np.float32)
    for S in (p.S, x2.shape[0]):
        assert wq.wq_describe_plan(I8, p.O, p.I, S).startswith("tiled"), S
    return p, x2


def test_tiled_calls_on_concurrent_streams():
    """Each stream has its own tiled workspace: calls queued on two streams with no ordering
    between them (different S, so different plane sizes) all equal their eager results."""
    p, x2h = _tiled_case(31)
    t = gu.upload(p)
    try:
        x1 = torch.from_numpy(p.x).cuda()
        x2 = torch.from_numpy(x2h).cuda()
        r1 = torch.empty((p.S, p.O), device="cuda")
        r2 = torch.empty((x2h.shape[0], p.O), device="cuda")
        gu.banner("concurrent streams: eager references")
        wq.wq_matmul_dev(t, x1, r1)
        wq.wq_matmul_dev(t, x2, r2)
        torch.cuda.synchronize()
        rows = np.arange(0, p.O, 29)
        for r, xh in ((r1, p.x), (r2, x2h)):
            y_ref, A = oracle.matmul_rows(I8, p.w, p.scales, xh, rows)
            gu.assert_within_bound(r.cpu().numpy()[:, rows], y_ref, A, "eager")
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        n = 12
        o1 = [torch.full_like(r1, float("nan")) for _ in range(n)]
        o2 = [torch.full_like(r2, float("nan")) for _ in range(n)]
        torch.cuda.synchronize()
        gu.banner("concurrent streams: %d calls on each of two streams" % n)
        for i in range(n):
            wq.wq_matmul_dev(t, x1, o1[i], stream=s1)
            wq.wq_matmul_dev(t, x2, o2[i], stream=s2)
        torch.cuda.synchronize()
        for i in range(n):
            assert torch.equal(o1[i], r1), "stream 1, call %d" % i
            assert torch.equal(o2[i], r2), "stream 2, call %d" % i
    finally:
        wq.wq_tensor_free(t)


def test_more_streams_than_workspaces():
    """Ten streams in turn, three rounds: from the ninth stream on, a stream takes over the least
    recently used stream's workspace; every result still equals the eager one."""
    p, x2h = _tiled_case(33)
    t = gu.upload(p)
    try:
        xs = [torch.from_numpy(p.x).cuda(), torch.from_numpy(x2h).cuda()]
        refs = [torch.empty((x.shape[0], p.O), device="cuda") for x in xs]
        gu.banner("ten streams: eager references")
        for x, r in zip(xs, refs):
            wq.wq_matmul_dev(t, x, r)
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream() for _ in range(10)]
        assert len({s.cuda_stream for s in streams}) == 10
        outs = []
        gu.banner("ten streams: three rounds")
        for rnd in range(3):
            for k, s in enumerate(streams):
                j = (k + rnd) % 2
                o = torch.full_like(refs[j], float("nan"))
                wq.wq_matmul_dev(t, xs[j], o, stream=s)
                outs.append((j, o))
        torch.cuda.synchronize()
        for i, (j, o) in enumerate(outs):
            assert torch.equal(o, refs[j]), "call %d" % i
    finally:
        wq.wq_tensor_free(t)


@pytest.mark.parametrize("mode,shape", [("bf16x3", "128x96x64"), ("bf16x3", "128x96x128"), ("bf16x3", "64x64x64"),
                                        ("bf16x3", "16x128x64"), ("bf16x3", "64x192x64"),
                                        ("fp32", "128x96x32"), ("fp32", "64x64x32")])
@pytest.mark.parametrize("fmt,O,I,S", [(I8, 200, 700, 150), (I4, 97, 2100, 20), (I2, 130, 4500, 70)])
def test_forced_tile_shapes(mode, shape, fmt, O, I, S):
    p = synth.ragged(fmt, O, I, S, seed=23 + O + S)
    t = gu.upload(p)
    try:
        gu.reinit_with_env(WQ_FORCE_PATH="tiled", WQ_TILED_MODE=mode, WQ_TILED_SHAPE=shape)
        plan = wq.wq_describe_plan(fmt, O, I, S)
        bm, bn, bk = shape.split("x")
        assert "mode=%s bm=%s bn=%s bk=%s" % (mode, bm, bn, bk) in plan, plan
        gu.banner("forced shape " + plan)
        y = gu.run_dev(t, p.x)
    finally:
        wq.wq_tensor_free(t)
        gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_TILED_MODE=None, WQ_TILED_SHAPE=None)
    y_ref, A = oracle.matmul(fmt, p.w, p.scales, p.x)
    gu.assert_within_bound(y, y_ref, A, "shape " + shape)
