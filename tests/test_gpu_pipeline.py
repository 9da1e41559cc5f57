"""GPU parity of the stream-ordered, device-resident feed-forward pipeline with host
input and output every step (the arrangement behind colibri docs "CUDA backend
(Linux)", section "The GPU-resident pipeline": activations stay on the device between
matmuls, and only the layer's input and output cross the bus).

Each step copies a fresh input for every expert from pinned host memory to the device,
runs the gated gate/up launch and the grouped down launch (wq_swiglu_ffn_dev), and
copies y back to pinned host memory, all queued without host synchronisation. Two
arrangements are captured into one HIP graph each and replayed: serialised on one
stream, and double-buffered with the copies on two copy streams overlapping the
compute (cross-stream events order the buffers). Every step's y, read back through
the host, must meet the oracle chain's bound (gate, up -> silu(g)*u -> down), and the
two arrangements must agree bit for bit.
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

E, S, HID, INTER, K = 3, 2, 1024, 384, 5


@pytest.fixture(scope="module")
def layer():
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_TILED_MODE=None, WQ_TILED_SHAPE=None)
    probs = synth.moe_decode(n_experts=E, S=S, hidden=HID, inter=INTER)
    ts = [gu.upload(p) for p in probs]
    gated = wq.wq_swiglu_create(ts[0::3], ts[1::3])
    down = wq.wq_grouped_create(ts[2::3])
    g = synth.rng(17000)
    x_steps = g.standard_normal((K, E, S, HID), dtype=np.float32)
    yield probs, gated, down, x_steps
    wq.wq_grouped_free(gated)
    wq.wq_grouped_free(down)
    for t in ts:
        wq.wq_tensor_free(t)


def _oracle_step(probs, x):
    """y of every expert for inputs x [E, S, HID], with the tolerance inputs."""
    out = []
    for e in range(E):
        gp, up, dp = probs[3 * e:3 * e + 3]
        gv, ag = oracle.matmul(gp.fmt, gp.w, gp.scales, x[e])
        uv, au = oracle.matmul(up.fmt, up.w, up.scales, x[e])
        h = oracle.silu_mul(gv, uv)
        y, _ = oracle.matmul(dp.fmt, dp.w, dp.scales, h)
        ref = {"g": gv, "Ag": ag, "u": uv, "Au": au, "h": h}
        out.append((ref, gu.h_bound(gv, ag, uv, au, h), y))
    return out


def _run(arrangement, gated, down, x_steps):
    dev = torch.device("cuda:%d" % gu.DEV)
    x_host = torch.empty((K, E, S, HID), dtype=torch.float32, pin_memory=True)
    x_host.copy_(torch.from_numpy(x_steps))
    y_host = torch.full((K, E, S, HID), float("nan"), dtype=torch.float32, pin_memory=True)
    xd = [torch.zeros((E, S, HID), device=dev) for _ in range(2)]
    hd = [torch.empty((E, S, INTER), device=dev) for _ in range(2)]
    yd = [torch.empty((E, S, HID), device=dev) for _ in range(2)]
    cin, cout = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    ev_in = [torch.cuda.Event() for _ in range(2)]
    ev_done = [torch.cuda.Event() for _ in range(2)]
    ev_out = [torch.cuda.Event() for _ in range(2)]

    def ffn(b, comp):
        wq.wq_swiglu_ffn_dev(gated, down, list(xd[b]), list(hd[b]), list(yd[b]), stream=comp)

    def serialised(comp):
        for t in range(K):
            xd[0].copy_(x_host[t], non_blocking=True)
            ffn(0, comp)
            y_host[t].copy_(yd[0], non_blocking=True)

    def overlapped(comp):
        fork = torch.cuda.Event()
        fork.record(comp)
        cin.wait_event(fork)
        cout.wait_event(fork)

        def load(t):
            b = t % 2
            with torch.cuda.stream(cin):
                if t >= 2:
                    cin.wait_event(ev_done[b])  # step t - 2 has read slot b
                xd[b].copy_(x_host[t], non_blocking=True)
                ev_in[b].record(cin)
        load(0)
        for t in range(K):
            b = t % 2
            if t + 1 < K:
                load(t + 1)
            comp.wait_event(ev_in[b])
            if t >= 2:
                comp.wait_event(ev_out[b])  # y of step t - 2 has left slot b
            ffn(b, comp)
            ev_done[b].record(comp)
            with torch.cuda.stream(cout):
                cout.wait_event(ev_done[b])
                y_host[t].copy_(yd[b], non_blocking=True)
                ev_out[b].record(cout)
        comp.wait_event(ev_out[(K - 1) % 2])  # join the output stream

    body = serialised if arrangement == "serialised" else overlapped
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    gu.banner("pipeline %s: capture" % arrangement)
    with torch.cuda.graph(g, stream=side):
        body(side)
    torch.cuda.synchronize()
    outs = []
    for rep in range(2):  # replays, with eager work between them
        y_host.fill_(float("nan"))
        gu.banner("pipeline %s: replay %d" % (arrangement, rep))
        g.replay()
        torch.cuda.synchronize()
        outs.append(y_host.numpy().copy())
        ffn(0, torch.cuda.current_stream())
        torch.cuda.synchronize()
    del g
    return outs


def test_pipeline_host_io_matches_oracle_every_step(layer):
    probs, gated, down, x_steps = layer
    refs = [_oracle_step(probs, x_steps[t]) for t in range(K)]
    results = {}
    for arrangement in ("serialised", "overlapped"):
        outs = _run(arrangement, gated, down, x_steps)
        np.testing.assert_array_equal(outs[0], outs[1])  # replays agree
        for t in range(K):
            for e in range(E):
                ref, bh, y_ref = refs[t][e]
                dp = probs[3 * e + 2]
                gu.assert_y(outs[0][t, e], dp.fmt, dp.w, dp.scales, ref["h"], bh, y_ref,
                            "%s step %d expert %d" % (arrangement, t, e))
        results[arrangement] = outs[0]
    np.testing.assert_array_equal(results["serialised"], results["overlapped"])
