"""Python binding of libwqmm.so, the weight-resident quantized matmul for MI355X.

    y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]

(colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四; colibri-analysis
"CUDA 后端", section 1.) Every function here has the name of the C entry point
it wraps (include/wqmm.h) and only marshals arguments: numpy arrays for host
buffers, torch tensors for device buffers and the current torch stream.
All computation happens in the HIP kernels of libwqmm.so; there is no CPU
fallback. A non-zero status becomes a WqError carrying the code.

The library is loaded after torch so that both use the same HIP runtime.
If libwqmm.so has not been built yet it is built once with hipcc; if that is
impossible the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

try:  # torch first: its HIP runtime is the one the library must bind to
    import torch
except ImportError:  # pragma: no cover - host-only use (plan description, row bytes)
    torch = None

WQ_F32, WQ_I8, WQ_I4, WQ_I2 = 0, 1, 2, 3
WQ_OK = 0
WQ_E_INVAL = -1
WQ_E_NODEV = -2
WQ_E_NOTINIT = -3
WQ_E_OOM = -4
WQ_E_MISMATCH = -5
WQ_E_HIP = -6
WQ_E_FAULT = -7
WQ_E_UNSUPPORTED = -8
WQ_MAX_DEVICES = 16
WQ_GEMV_MAX_S = 8

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwqmm.so")

_c_int_p = ctypes.POINTER(ctypes.c_int)
_c_size_p = ctypes.POINTER(ctypes.c_size_t)


class WqError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (what, wq_strerror(code), code))


def _bind(lib):
    vp, ci, cl = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
    sig = {
        "wq_init": (ci, [_c_int_p, ci]),
        "wq_mem_info": (ci, [ci, _c_size_p, _c_size_p]),
        "wq_row_bytes": (cl, [ci, cl]),
        "wq_tensor_upload": (ci, [ctypes.POINTER(vp), ci, ci, ci, ci, vp, vp]),
        "wq_tensor_upload_gs": (ci, [ctypes.POINTER(vp), ci, ci, ci, ci, ci, vp, vp]),
        "wq_matmul": (ci, [ctypes.POINTER(vp), ci, ci, ci, ci, vp, vp, vp, ci, vp]),
        "wq_matmul_t": (ci, [vp, vp, ci, vp]),
        "wq_matmul_dev": (ci, [vp, vp, ci, vp, vp]),
        "wq_grouped_create": (ci, [ctypes.POINTER(vp), ci, ctypes.POINTER(vp)]),
        "wq_grouped_matmul_dev": (ci, [vp, ctypes.POINTER(vp), _c_int_p, ctypes.POINTER(vp), vp]),
        "wq_grouped_free": (ci, [vp]),
        "wq_swiglu_create": (ci, [ctypes.POINTER(vp), ctypes.POINTER(vp), ci, ctypes.POINTER(vp)]),
        "wq_swiglu_matmul_dev": (ci, [vp, ctypes.POINTER(vp), _c_int_p, ctypes.POINTER(vp), vp]),
        "wq_swiglu_ffn_dev": (ci, [vp, vp, ctypes.POINTER(vp), _c_int_p, ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), vp]),
        "wq_tensor_free": (ci, [vp]),
        "wq_strerror": (ctypes.c_char_p, [ci]),
        "wq_describe_plan": (ci, [ci, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t]),
        "wq_describe_plan_gs": (ci, [ci, ci, ci, ci, ci, ctypes.c_char_p, ctypes.c_size_t]),
        "wq_stream_read_dev": (ci, [vp, ctypes.c_size_t, ci, ci, vp, vp]),
        "wq_matmul_dev_noalloc": (ci, [vp, vp, ci, vp, vp]),
        "wq_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def _load():
    if not os.path.exists(LIB_PATH):
        from . import build as _build  # nothing built yet: build once, in-tree
        _build.build()
    return _bind(ctypes.CDLL(LIB_PATH))


lib = _load()


def _check(rc: int, what: str):
    if rc != WQ_OK:
        raise WqError(rc, what)


def _stream_handle(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _host_f32(a, shape, what):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.shape != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (what, tuple(shape), a.shape))
    return a


def _dev_f32(t, shape, device, what):
    if torch is None or not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor on a GPU" % what)
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 GPU tensor" % what)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (what, tuple(shape), tuple(t.shape)))
    if t.device.index != device:
        raise ValueError("%s is on %s, tensor lives on cuda:%d" % (what, t.device, device))
    return ctypes.c_void_p(t.data_ptr())


class Tensor:
    """Handle of a resident weight tensor (the C wq_tensor*)."""

    def __init__(self, ptr: ctypes.c_void_p, device: int, fmt: int, O: int, I: int):
        self.ptr, self.device, self.fmt, self.O, self.I = ptr, device, fmt, O, I

    def __repr__(self):
        return "Tensor(device=%d, fmt=%d, O=%d, I=%d)" % (self.device, self.fmt, self.O, self.I)


class Group:
    """Handle of a tensor group (the C wq_group*); `ups` is set for a gated group."""

    def __init__(self, ptr: ctypes.c_void_p, tensors, ups=None):
        self.ptr, self.tensors = ptr, list(tensors)
        self.ups = None if ups is None else list(ups)


# ----------------------------------------------------------------------------
# C ABI wrappers


def wq_strerror(code: int) -> str:
    return lib.wq_strerror(int(code)).decode()


def wq_init(devices=None) -> None:
    if devices is None:
        _check(lib.wq_init(None, 0), "wq_init")
        return
    devs = list(devices)
    arr = (ctypes.c_int * max(1, len(devs)))(*devs)
    _check(lib.wq_init(arr, len(devs)), "wq_init")


def wq_mem_info(device: int = 0):
    f, t = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.wq_mem_info(int(device), ctypes.byref(f), ctypes.byref(t)), "wq_mem_info")
    return f.value, t.value


def wq_row_bytes(fmt: int, I: int) -> int:
    return int(lib.wq_row_bytes(int(fmt), int(I)))


def _weights(fmt, O, I, w, scales):
    rb = wq_row_bytes(fmt, I)
    if rb < 0:
        raise WqError(WQ_E_INVAL, "wq_row_bytes")
    w = np.ascontiguousarray(w, dtype=np.uint8)
    if w.size != O * rb:
        raise ValueError("w must hold O * row_bytes = %d bytes, got %d" % (O * rb, w.size))
    if scales is not None:
        scales = _host_f32(scales, (O,), "scales")
    return w, scales


def wq_tensor_upload(t, device: int, fmt: int, O: int, I: int, w, scales) -> Tensor:
    """Upload (t is None) or validate (t given) a resident tensor; returns the handle."""
    h = ctypes.c_void_p(t.ptr.value if t is not None else None)
    if t is None:
        w, scales = _weights(fmt, O, I, w, scales)
        wp, sp = w.ctypes.data, (scales.ctypes.data if scales is not None else None)
    else:
        wp, sp = None, None
    _check(lib.wq_tensor_upload(ctypes.byref(h), int(device), int(fmt), int(O), int(I), wp, sp),
           "wq_tensor_upload")
    return t if t is not None else Tensor(h, int(device), int(fmt), int(O), int(I))


def wq_tensor_upload_gs(t, device: int, fmt: int, O: int, I: int, gs: int, w, scales) -> Tensor:
    """Upload with group-wise scales (scales float32 [O, ceil(I/gs)]) or validate; returns the handle."""
    h = ctypes.c_void_p(t.ptr.value if t is not None else None)
    if t is None:
        w, _ = _weights(fmt, O, I, w, None)
        ng = (int(I) + int(gs) - 1) // int(gs) if int(gs) > 0 else 1
        scales = _host_f32(scales, (O, ng), "scales")
        wp, sp = w.ctypes.data, scales.ctypes.data
    else:
        wp, sp = None, None
    _check(lib.wq_tensor_upload_gs(ctypes.byref(h), int(device), int(fmt), int(O), int(I), int(gs), wp, sp),
           "wq_tensor_upload_gs")
    return t if t is not None else Tensor(h, int(device), int(fmt), int(O), int(I))


def wq_matmul(t, device: int, fmt: int, O: int, I: int, w, scales, x):
    """Lazy upload + synchronous host matmul; returns (handle, y [S, O])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] != I:
        raise ValueError("x must be [S, I]")
    S = x.shape[0]
    y = np.empty((S, O), dtype=np.float32)
    h = ctypes.c_void_p(t.ptr.value if t is not None else None)
    if t is None:
        w, scales = _weights(fmt, O, I, w, scales)
        wp, sp = w.ctypes.data, (scales.ctypes.data if scales is not None else None)
    else:
        wp, sp = None, None
    _check(lib.wq_matmul(ctypes.byref(h), int(device), int(fmt), int(O), int(I), wp, sp,
                         x.ctypes.data, S, y.ctypes.data), "wq_matmul")
    return (t if t is not None else Tensor(h, int(device), int(fmt), int(O), int(I))), y


def wq_matmul_t(t: Tensor, x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] != t.I:
        raise ValueError("x must be [S, I]")
    y = np.empty((x.shape[0], t.O), dtype=np.float32)
    _check(lib.wq_matmul_t(t.ptr, x.ctypes.data, x.shape[0], y.ctypes.data), "wq_matmul_t")
    return y


def wq_matmul_dev(t: Tensor, x_dev, y_dev, stream=None) -> None:
    """y_dev[S, O] = matmul(t, x_dev[S, I]) as one launch on `stream` (default: current)."""
    S = x_dev.shape[0] if x_dev.dim() == 2 else -1
    xp = _dev_f32(x_dev, (S, t.I), t.device, "x_dev")
    yp = _dev_f32(y_dev, (S, t.O), t.device, "y_dev")
    _check(lib.wq_matmul_dev(t.ptr, xp, int(S), yp, _stream_handle(stream, t.device)), "wq_matmul_dev")


def wq_matmul_dev_noalloc(t: Tensor, x_dev, y_dev, stream=None) -> None:
    """As wq_matmul_dev, allocating nothing (the tiled workspace is the library's fixed
    per-device array of wq_noalloc_scratch_bytes() bytes)."""
    S = x_dev.shape[0] if x_dev.dim() == 2 else -1
    xp = _dev_f32(x_dev, (S, t.I), t.device, "x_dev")
    yp = _dev_f32(y_dev, (S, t.O), t.device, "y_dev")
    _check(lib.wq_matmul_dev_noalloc(t.ptr, xp, int(S), yp, _stream_handle(stream, t.device)),
           "wq_matmul_dev_noalloc")


def wq_noalloc_scratch_bytes() -> int:
    return int(lib.wq_noalloc_scratch_bytes())


def wq_grouped_create(tensors) -> Group:
    ts = list(tensors)
    arr = (ctypes.c_void_p * len(ts))(*[t.ptr.value for t in ts])
    h = ctypes.c_void_p(None)
    _check(lib.wq_grouped_create(arr, len(ts), ctypes.byref(h)), "wq_grouped_create")
    return Group(h, ts)


def wq_grouped_matmul_dev(g: Group, xs, ys, stream=None) -> None:
    """For each g: ys[g][S_g, O_g] = matmul(tensor g, xs[g][S_g, I_g]); xs[g] None means S_g = 0."""
    G = len(g.tensors)
    if len(xs) != G or len(ys) != G:
        raise ValueError("need one x and one y per tensor")
    xp = (ctypes.c_void_p * G)()
    yp = (ctypes.c_void_p * G)()
    Ss = (ctypes.c_int * G)()
    for i, (t, x, y) in enumerate(zip(g.tensors, xs, ys)):
        if x is None:
            Ss[i] = 0
            continue
        S = x.shape[0]
        xp[i] = _dev_f32(x, (S, t.I), t.device, "xs[%d]" % i).value
        yp[i] = _dev_f32(y, (S, t.O), t.device, "ys[%d]" % i).value
        Ss[i] = S
    dev = g.tensors[0].device
    _check(lib.wq_grouped_matmul_dev(g.ptr, xp, Ss, yp, _stream_handle(stream, dev)), "wq_grouped_matmul_dev")


def _per_problem(tensors, xs, outs, out_cols, what):
    G = len(tensors)
    if len(xs) != G or len(outs) != G:
        raise ValueError("need one x and one %s per problem" % what)
    xp = (ctypes.c_void_p * G)()
    op = (ctypes.c_void_p * G)()
    Ss = (ctypes.c_int * G)()
    for i, (t, x, o) in enumerate(zip(tensors, xs, outs)):
        if x is None:
            Ss[i] = 0
            continue
        S = x.shape[0]
        xp[i] = _dev_f32(x, (S, t.I), t.device, "xs[%d]" % i).value
        op[i] = _dev_f32(o, (S, out_cols[i]), t.device, "%s[%d]" % (what, i)).value
        Ss[i] = S
    return xp, Ss, op


def wq_swiglu_create(gates, ups) -> Group:
    """Gated group: expert e pairs gates[e] with ups[e] (same shape)."""
    gs, us = list(gates), list(ups)
    if len(gs) != len(us):
        raise ValueError("need one up tensor per gate tensor")
    ga = (ctypes.c_void_p * len(gs))(*[t.ptr.value for t in gs])
    ua = (ctypes.c_void_p * len(us))(*[t.ptr.value for t in us])
    h = ctypes.c_void_p(None)
    _check(lib.wq_swiglu_create(ga, ua, len(gs), ctypes.byref(h)), "wq_swiglu_create")
    return Group(h, gs, us)


def wq_swiglu_matmul_dev(g: Group, xs, hs, stream=None) -> None:
    """hs[e][S_e, O_e] = silu(gate_e . xs[e]) * (up_e . xs[e]); xs[e] None skips expert e."""
    xp, Ss, hp = _per_problem(g.tensors, xs, hs, [t.O for t in g.tensors], "hs")
    dev = g.tensors[0].device
    _check(lib.wq_swiglu_matmul_dev(g.ptr, xp, Ss, hp, _stream_handle(stream, dev)), "wq_swiglu_matmul_dev")


def wq_swiglu_ffn_dev(g: Group, down: Group, xs, hs, ys, stream=None) -> None:
    """Both halves of the gated feed-forward: hs as wq_swiglu_matmul_dev, then ys[e] = down_e . hs[e]."""
    xp, Ss, hp = _per_problem(g.tensors, xs, hs, [t.O for t in g.tensors], "hs")
    if len(ys) != len(down.tensors):
        raise ValueError("need one y per expert")
    E = len(g.tensors)
    yp = (ctypes.c_void_p * E)()
    for i in range(E):
        if Ss[i] > 0:
            t = down.tensors[i]
            yp[i] = _dev_f32(ys[i], (Ss[i], t.O), t.device, "ys[%d]" % i).value
    dev = g.tensors[0].device
    _check(lib.wq_swiglu_ffn_dev(g.ptr, down.ptr, xp, Ss, hp, yp, _stream_handle(stream, dev)),
           "wq_swiglu_ffn_dev")


def wq_grouped_free(g: Group) -> None:
    _check(lib.wq_grouped_free(g.ptr), "wq_grouped_free")
    g.ptr = ctypes.c_void_p(None)


def wq_tensor_free(t: Tensor) -> None:
    if t is None:
        return
    _check(lib.wq_tensor_free(t.ptr), "wq_tensor_free")
    t.ptr = ctypes.c_void_p(None)


def wq_describe_plan(fmt: int, O: int, I: int, S: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib.wq_describe_plan(int(fmt), int(O), int(I), int(S), buf, 256), "wq_describe_plan")
    return buf.value.decode()


def wq_describe_plan_gs(fmt: int, O: int, I: int, S: int, gs: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib.wq_describe_plan_gs(int(fmt), int(O), int(I), int(S), int(gs), buf, 256), "wq_describe_plan_gs")
    return buf.value.decode()


def wq_stream_read_dev(buf_dev, waves: int, loads_in_flight: int, out_dev, stream=None) -> None:
    """Read every byte of the device tensor buf_dev once (HBM read ceiling);
    out_dev: int32 device tensor of >= 64 * waves elements."""
    nbytes = buf_dev.numel() * buf_dev.element_size()
    if not buf_dev.is_cuda or not buf_dev.is_contiguous() or not out_dev.is_cuda:
        raise ValueError("device tensors expected")
    if out_dev.numel() * out_dev.element_size() < 4 * 64 * int(waves):
        raise ValueError("out_dev too small")
    _check(lib.wq_stream_read_dev(ctypes.c_void_p(buf_dev.data_ptr()), nbytes, int(waves), int(loads_in_flight),
                                  ctypes.c_void_p(out_dev.data_ptr()), _stream_handle(stream, buf_dev.device)),
           "wq_stream_read_dev")
