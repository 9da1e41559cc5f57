"""Helpers for the GPU parity tests: device buffers with canaries, the bound check."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import weight_only_quantized_matmul_amd as wq

DEV = 0
CANARY = np.float32(-1.2345678e-33).view(np.uint32)  # unlikely bit pattern, finite
GUARD = 256  # floats of canary before and after every output


def banner(msg: str):
    """Name the case on stdout before a GPU step, flushed, so a fault report says where."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def init():
    wq.wq_init([DEV])


def reinit_with_env(**env):
    """Set WQ_* knobs (None removes one) and re-read them in the library."""
    for k, v in env.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = str(v)
    wq.wq_init([DEV])


def upload(p):
    return wq.wq_tensor_upload(None, DEV, p.fmt, p.O, p.I, p.w, p.scales)


def guarded_output(S: int, O: int):
    """(buffer, y view [S, O]); the view is surrounded by GUARD canary floats."""
    buf = torch.empty(S * O + 2 * GUARD, dtype=torch.int32, device="cuda:%d" % DEV)
    buf.fill_(int(np.int32(CANARY.view(np.int32))))
    y = buf[GUARD:GUARD + S * O].view(torch.float32).view(S, O)
    return buf, y


def check_canaries(buf, S: int, O: int):
    h = buf.cpu().numpy().view(np.uint32)
    assert np.all(h[:GUARD] == CANARY), "write before the output buffer"
    assert np.all(h[GUARD + S * O:] == CANARY), "write past the output buffer"


def run_dev(t, x: np.ndarray, stream=None, x_offset: int = 0) -> np.ndarray:
    """wq_matmul_dev on device copies of x; checks the canaries; returns y on the host.

    x_offset > 0 places x at that many floats into a larger buffer (misaligned start).
    """
    S = x.shape[0]
    xb = torch.zeros(x.size + x_offset, dtype=torch.float32, device="cuda:%d" % DEV)
    xb[x_offset:] = torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).to(xb.device)
    xd = xb[x_offset:].view(S, x.shape[1])
    buf, y = guarded_output(S, t.O)
    wq.wq_matmul_dev(t, xd, y, stream=stream)
    torch.cuda.synchronize()
    check_canaries(buf, S, t.O)
    return y.cpu().numpy().copy()


def bound_ratio(y: np.ndarray, y_ref: np.ndarray, A: np.ndarray) -> float:
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    return float(np.max(err / (1e-5 * A + 1e-30))) if err.size else 0.0


def assert_within_bound(y, y_ref, A, what=""):
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    bound = 1e-5 * A + 1e-30
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements outside |y-y_ref| <= 1e-5*A + 1e-30; first %s; "
                             "worst err/bound %.3g" % (what, int(bad.sum()), bad.size, idx.tolist(),
                                                        float(np.max(err / bound))))


# ---------------------------------------------------------------------------------------
# gated feed-forward: tolerance of h = silu(g) * u derived from the matmul contract
# (|g - g_ref| <= Eg = 1e-5*Ag + ulp(g_ref) + 1e-30, the same for u) and silu's slope,
# which never exceeds 1.1 in magnitude; 2e-6 relative covers the fp32 evaluation of
# silu and the product (a few ulps).


def silu64(z):
    z = z.astype(np.float64)
    return z / (1.0 + np.exp(-z))


def ulp32(v):
    return np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)


def h_bound(g, Ag, u, Au, h):
    Eg = 1e-5 * Ag + ulp32(g) + 1e-30
    Eu = 1e-5 * Au + ulp32(u) + 1e-30
    t = 1.1 * Eg * (np.abs(u) + Eu) + np.abs(silu64(g)) * Eu
    return t + 2e-6 * (np.abs(h).astype(np.float64) + t) + 1e-30


def assert_y(y, fmt_dn, dw, dsc, ref_h, bh, y_ref, what):
    """Down projection of h: |y - y_ref| <= 1e-5*A_down(|h_ref| + Bh) + A_down(Bh) + ulp(y_ref)
    + 1e-30, A_down(v)[o] = sum_i |scale[o]*q[o,i]|*v[i] (the oracle's bound magnitude on a
    non-negative input v)."""
    import oracle
    _, a1 = oracle.matmul(fmt_dn, dw, dsc, (np.abs(ref_h).astype(np.float64) + bh).astype(np.float32))
    _, a2 = oracle.matmul(fmt_dn, dw, dsc, bh.astype(np.float32))
    by = 1e-5 * a1 + 1.0001 * a2 + ulp32(y_ref) + 1e-30
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    bad = err > by
    assert not bad.any(), "%s: %d of %d y elements out of bound; worst err/bound %.3g" % (
        what, int(bad.sum()), bad.size, float(np.max(err / by)))


def assert_h(h, ref, what):
    bh = h_bound(ref["g"], ref["Ag"], ref["u"], ref["Au"], ref["h"])
    err = np.abs(h.astype(np.float64) - ref["h"].astype(np.float64))
    assert np.all(np.isfinite(h)), what
    bad = err > bh
    assert not bad.any(), "%s: %d of %d h elements out of bound; worst err/bound %.3g at %s" % (
        what, int(bad.sum()), bad.size, float(np.max(err / bh)), np.argwhere(bad)[:3].tolist())
    return bh


# ---------------------------------------------------------------------------------------
# launch counting: capture a call into a HIP graph and count its kernel nodes


def _hip():
    import ctypes
    lib = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has already loaded
    lib.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    lib.hipGraphGetNodes.restype = ctypes.c_int
    lib.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    lib.hipGraphNodeGetType.restype = ctypes.c_int
    return lib


def count_kernel_launches(fn) -> int:
    """Kernel nodes recorded when fn() runs under stream capture (fn must launch on the
    current stream and allocate nothing); the captured graph is not replayed."""
    import ctypes
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    hip = _hip()
    graph = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    kernels = 0
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        kernels += int(t.value == 0)  # hipGraphNodeTypeKernel
    del g
    return kernels
