"""GPU parity of the gated feed-forward calls (wq_swiglu_matmul_dev,
wq_swiglu_ffn_dev) against the oracle's matmul + silu_mul chain, through the
C ABI.

Tolerance, derived from the matmul contract (|g - g_ref| <= Eg = 1e-5*Ag +
ulp(g_ref) + 1e-30, the same for u) and silu's slope, which never exceeds
1.1 in magnitude:

    |h - h_ref| <= Bh = 1.1*Eg*(|u_ref| + Eu) + |silu(g_ref)|*Eu
                       + 2e-6*(|h_ref| + those terms) + 1e-30

(2e-6 relative covers the fp32 evaluation of silu and the product: a few
ulps). The down projection then meets

    |y - y_ref| <= 1e-5*A_down(|h_ref| + Bh) + A_down(Bh) + ulp(y_ref) + 1e-30,

A_down(v)[o] = sum_i |scale[o]*q[o,i]|*v[i], which the oracle's bound
magnitude gives for a non-negative input v.
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

F32, I8, I4, I2 = 0, 1, 2, 3


@pytest.fixture(scope="module", autouse=True)
def device():
    gu.reinit_with_env(WQ_FORCE_PATH=None, WQ_GEMV_MAX_S=None, WQ_TILED_MODE=None, WQ_TILED_SHAPE=None)
    yield
    gu.reinit_with_env(WQ_FORCE_PATH=None)


silu64, ulp32, h_bound, assert_h = gu.silu64, gu.ulp32, gu.h_bound, gu.assert_h


assert_y = gu.assert_y


class Expert:
    def __init__(self, fmt, O, I, S, seed, gs=0, down_fmt=None, down_O=None):
        g = synth.rng(seed)
        self.fmt, self.O, self.I, self.S, self.gs = fmt, O, I, S, gs
        self.gw = synth.weights(g, fmt, O, I)
        self.uw = synth.weights(g, fmt, O, I)
        if gs:
            ng = oracle.n_groups(I, gs)
            self.gsc = g.uniform(0.002, 0.05, size=(O, ng)).astype(np.float32)
            self.usc = g.uniform(0.002, 0.05, size=(O, ng)).astype(np.float32)
        else:
            self.gsc = synth.scales(g, O, 0.002, 0.05)
            self.usc = synth.scales(g, O, 0.002, 0.05)
        self.x = synth.activations(g, S, I)
        self.dfmt = fmt if down_fmt is None else down_fmt
        self.dO = down_O or I
        self.dw = synth.weights(g, self.dfmt, self.dO, O)
        self.dsc = synth.scales(g, self.dO, 0.002, 0.05)

    def upload(self):
        if self.gs:
            gt = wq.wq_tensor_upload_gs(None, gu.DEV, self.fmt, self.O, self.I, self.gs, self.gw, self.gsc)
            ut = wq.wq_tensor_upload_gs(None, gu.DEV, self.fmt, self.O, self.I, self.gs, self.uw, self.usc)
        else:
            gt = wq.wq_tensor_upload(None, gu.DEV, self.fmt, self.O, self.I, self.gw, self.gsc)
            ut = wq.wq_tensor_upload(None, gu.DEV, self.fmt, self.O, self.I, self.uw, self.usc)
        dt = wq.wq_tensor_upload(None, gu.DEV, self.dfmt, self.dO, self.O, self.dw, self.dsc)
        return gt, ut, dt

    def reference(self):
        if self.gs:
            g, ag = oracle.matmul_gs(self.fmt, self.gw, self.gsc, self.gs, self.x)
            u, au = oracle.matmul_gs(self.fmt, self.uw, self.usc, self.gs, self.x)
        else:
            g, ag = oracle.matmul(self.fmt, self.gw, self.gsc, self.x)
            u, au = oracle.matmul(self.fmt, self.uw, self.usc, self.x)
        h = oracle.silu_mul(g, u)
        y, ay = oracle.matmul(self.dfmt, self.dw, self.dsc, h)
        return {"g": g, "Ag": ag, "u": u, "Au": au, "h": h, "y": y, "Ay": ay}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:%d" % gu.DEV)


def run_chain(experts, with_down=True, what="swiglu"):
    """Upload, run the gated calls, compare h (and y) with the oracle for every expert."""
    ts = [e.upload() for e in experts]
    grp = wq.wq_swiglu_create([t[0] for t in ts], [t[1] for t in ts])
    down = wq.wq_grouped_create([t[2] for t in ts])
    try:
        xs = [dev(e.x) if e.S > 0 else None for e in experts]
        hbufs = [gu.guarded_output(max(e.S, 1), e.O) for e in experts]
        ybufs = [gu.guarded_output(max(e.S, 1), e.dO) for e in experts]
        hs = [hb[1] for hb in hbufs]
        ys = [yb[1] for yb in ybufs]
        gu.banner("%s E=%d shapes=%s" % (what, len(experts),
                                          [(e.fmt, e.O, e.I, e.S, e.gs) for e in experts]))
        if with_down:
            wq.wq_swiglu_ffn_dev(grp, down, xs, hs, ys)
        else:
            wq.wq_swiglu_matmul_dev(grp, xs, hs)
        torch.cuda.synchronize()
        out = []
        for i, e in enumerate(experts):
            gu.check_canaries(hbufs[i][0], max(e.S, 1), e.O)
            gu.check_canaries(ybufs[i][0], max(e.S, 1), e.dO)
            if e.S == 0:
                out.append(None)
                continue
            h = hs[i].cpu().numpy()
            ref = e.reference()
            bh = assert_h(h, ref, "%s expert %d h" % (what, i))
            y = None
            if with_down:
                y = ys[i].cpu().numpy()
                assert_y(y, e.dfmt, e.dw, e.dsc, ref["h"], bh, ref["y"], "%s expert %d y" % (what, i))
            out.append((h, y, ref))
        return out
    finally:
        wq.wq_grouped_free(grp)
        wq.wq_grouped_free(down)
        for t in ts:
            for x in t:
                wq.wq_tensor_free(x)


@pytest.mark.parametrize("fmt", [F32, I8, I4, I2])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 8, 9, 24])
def test_swiglu_parity_formats(fmt, S):
    # O ragged, I ragged: the one-launch, per-expert and composed forms by S
    experts = [Expert(fmt, 300, 1000, S, seed=9000 + 40 * fmt + S + 7 * k) for k in range(3)]
    run_chain(experts, what="fmt%d S%d" % (fmt, S))


@pytest.mark.parametrize("fmt,I,S", [(I4, 6144, 1), (I4, 6144, 2), (I4, 6144, 4), (I8, 6144, 1),
                                     (I8, 6144, 3), (I2, 8192, 2), (I2, 12000, 8), (I8, 12000, 1)])
def test_swiglu_long_rows(fmt, I, S):
    # rows past one wave's coverage: each expert runs as a paired launch with
    # several waves per row
    experts = [Expert(fmt, 96, I, S, seed=9300 + I + S + k, down_O=128) for k in range(2)]
    run_chain(experts, what="long fmt%d I%d S%d" % (fmt, I, S))


def test_swiglu_mixed_S_and_skip():
    experts = [Expert(I4, 130, 640, S, seed=9400 + S) for S in (1, 0, 3, 2, 0, 1)]
    run_chain(experts, what="mixed")


def test_swiglu_many_experts_two_chunks():
    # 66 experts: more than one launch chunk of paired problems, rows of 1..3 slots
    g0 = synth.rng(9450)
    experts = [Expert(I4, int(g0.integers(1, 40)), int(g0.choice([64, 1500, 2100, 5000])), 1, seed=9460 + k,
                      down_O=32) for k in range(66)]
    run_chain(experts, what="66 experts")


def test_swiglu_group_scales():
    experts = [Expert(fmt, 200, 1024, S, seed=9500 + fmt + S, gs=128) for fmt, S in
               ((I8, 1), (I4, 2), (I2, 5))]
    for e in experts:
        run_chain([e], what="gs")


def test_swiglu_forced_tiled():
    gu.reinit_with_env(WQ_FORCE_PATH="tiled")
    try:
        run_chain([Expert(I4, 200, 700, S, seed=9600 + S) for S in (1, 3)], what="tiled")
    finally:
        gu.reinit_with_env(WQ_FORCE_PATH=None)


def test_swiglu_moe_decode_shape():
    # 8 experts, gate/up [2048, 6144] int4 and down [6144, 2048] int4, one row each
    experts = [Expert(I4, 2048, 6144, 1, seed=9700 + k) for k in range(8)]
    run_chain(experts, what="moe-decode")


def test_swiglu_moe_decode_shape_batched():
    experts = [Expert(I4, 2048, 6144, S, seed=9750 + S) for S in (2, 4, 8, 16)]
    run_chain(experts, what="moe-batched")


@pytest.mark.parametrize("E,S,launches", [(8, 8, 2), (20, 5, 3), (8, 24, 2)])
def test_swiglu_few_rows_grouped_launches(E, S, launches):
    """2..16 rows per expert: gate and up of up to 16 experts per few-rows
    launch, then one activation launch per 32 experts."""
    experts = [Expert(I4, 2048 if E == 8 else 130 + 7 * k, 6144 if E == 8 else 1000, S, seed=9800 + E + k,
                      down_O=256) for k in range(E)]
    ts = [e.upload() for e in experts]
    grp = wq.wq_swiglu_create([t[0] for t in ts], [t[1] for t in ts])
    try:
        xs = [dev(e.x) for e in experts]
        hs = [torch.empty((S, e.O), dtype=torch.float32, device="cuda:%d" % gu.DEV) for e in experts]
        gu.banner("swiglu grouped few rows E=%d S=%d" % (E, S))
        wq.wq_swiglu_matmul_dev(grp, xs, hs)  # eager first: the workspace then holds every u
        torch.cuda.synchronize()
        for i, e in enumerate(experts):
            assert_h(hs[i].cpu().numpy(), e.reference(), "expert %d h" % i)
        gu.banner("swiglu grouped few rows E=%d S=%d: launch count" % (E, S))
        assert gu.count_kernel_launches(lambda: wq.wq_swiglu_matmul_dev(grp, xs, hs)) == launches
    finally:
        wq.wq_grouped_free(grp)
        for t in ts:
            for x in t:
                wq.wq_tensor_free(x)


def test_swiglu_exact_zero_rows():
    # gate codes that all decode to 0 give g = 0 exactly, so h = 0; up codes
    # that decode to 0 give u = 0 and h = 0; a zero h gives y = 0 exactly
    for fmt, zero in ((I8, 0x00), (I4, 0x88), (I2, 0xAA)):
        e = Expert(fmt, 64, 512, 2, seed=9800 + fmt)
        e.gw[:20] = zero
        e.uw[20:40] = zero
        out = run_chain([e], what="zeros fmt%d" % fmt)
        h, y, _ = out[0]
        assert np.all(h[:, :40] == 0.0)
        e2 = Expert(fmt, 64, 512, 2, seed=9810 + fmt)
        e2.gw[:] = zero
        h2, y2, _ = run_chain([e2], what="all-zero gate fmt%d" % fmt)[0]
        assert np.all(h2 == 0.0) and np.all(y2 == 0.0)


def test_swiglu_rejects_bad_arguments():
    e = Expert(I4, 64, 256, 1, seed=9900)
    gt, ut, dt = e.upload()
    other = wq.wq_tensor_upload(None, gu.DEV, I4, 64, 512, synth.weights(synth.rng(1), I4, 64, 512),
                                synth.scales(synth.rng(2), 64, 0.01, 0.02))
    try:
        with pytest.raises(wq.WqError) as ei:
            wq.wq_swiglu_create([gt], [other])  # up of another shape
        assert ei.value.code == wq.WQ_E_INVAL
        grp = wq.wq_swiglu_create([gt], [ut])
        plain = wq.wq_grouped_create([dt])
        wrong_down = wq.wq_grouped_create([other])  # I = 512 != gate O = 64
        try:
            x = dev(e.x)
            h = torch.empty(1, 64, device=x.device)
            y = torch.empty(1, 256, device=x.device)
            L = wq.lib
            xp = (ctypes.c_void_p * 1)(x.data_ptr())
            hp = (ctypes.c_void_p * 1)(h.data_ptr())
            yp = (ctypes.c_void_p * 1)(y.data_ptr())
            S = (ctypes.c_int * 1)(1)
            # a gated group is not a plain group and vice versa
            assert L.wq_grouped_matmul_dev(grp.ptr, xp, S, hp, None) == wq.WQ_E_INVAL
            assert L.wq_swiglu_matmul_dev(plain.ptr, xp, S, hp, None) == wq.WQ_E_INVAL
            assert L.wq_swiglu_ffn_dev(grp.ptr, wrong_down.ptr, xp, S, hp, yp, None) == wq.WQ_E_INVAL
            assert L.wq_swiglu_ffn_dev(grp.ptr, grp.ptr, xp, S, hp, yp, None) == wq.WQ_E_INVAL
            neg = (ctypes.c_int * 1)(-1)
            assert L.wq_swiglu_matmul_dev(grp.ptr, xp, neg, hp, None) == wq.WQ_E_INVAL
        finally:
            wq.wq_grouped_free(grp)
            wq.wq_grouped_free(plain)
            wq.wq_grouped_free(wrong_down)
    finally:
        for t in (gt, ut, dt, other):
            wq.wq_tensor_free(t)
