#!/usr/bin/env python3
"""Benchmark of the weight-resident quantized matmul on one MI355X.

Default workload (the headline): int4 W [12288, 6144] (two codes per byte, low
nibble = even column, value = nibble - 8), per-row fp32 scales, fp32 x with
S = 1; one step = one y = matmul(W, x) over a weight copy already resident in
HBM. Weights rotate over >= 1 GiB of distinct copies so the 256 MB Infinity
Cache cannot serve them. K steps are captured into one HIP graph (one kernel
node per step) and replayed once inside the timed region; x and y stay on the
device.

Prints one JSON line: value = weight bytes streamed per second (GB/s) for the
GEMV workloads, GFLOP/s for the prefill workload; `roofline` compares the
dominant kernel's algorithmic bytes (or flops) per launch, divided by its
average launch duration from HIP events on the launch stream, with the MI355X
peak; `cpu_baseline` is the CPU oracle timed on this host on a bounded sample
of the same workload.

The moe_ffn workload runs the whole gated feed-forward of 8 int4 experts per
step (the fused gate/up launch writing h = silu(g) * u, then the grouped down
launch); its roofline is that of the gate/up launch, timed in a graph of its
own. moe_ffn_pipeline measures the same step and adds `config.pipeline`: the
per-step time with the activations device-resident (graph replay, eager
launches, a host synchronisation every step) and with host input/output
every step (serialised on one stream, or double-buffered on copy streams that
overlap the compute), the overlapped outputs checked against eager ones.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix
FP32_VALU_FMA_PEAK_TFLOPS = 78.6  # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (no packed FMA)
METRIC = "effective weight GB/s (and % of HBM peak) for S=1 int4 GEMV; GFLOP/s at S=512"
ROTATION_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="dense_gemv",
                    choices=["dense_gemv", "moe_decode", "moe_decode_s8", "moe_ffn", "moe_ffn_s8", "moe_ffn_pipeline", "int2_gemv_s1", "int2_gemv_s4", "int2_gemv_s8",
                             "int2_gemv_s2", "int2_gemv_s16", "dense_gemv_s2", "dense_gemv_s4", "dense_gemv_s8",
                             "dense_gemv_s16", "dense_gemv_gs128", "dense_gemv_s8_gs128", "prefill_gs128",
                             "prefill"])
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the stream-read ceiling measured beside HBM-bound workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (10 times) for counter calibration")
    return ap.parse_args()


COUNTER_SUMMARY = {"dense_gemv": "profiles/gemv_int4_dense_gemv_hbm_counters.txt"}


# sources the counted kernel is compiled from (the register GEMV)
COUNTED_SOURCES = ("gemv_kernels.hip", "wq_internal.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in COUNTED_SOURCES:
        with open(os.path.join(ROOT, "weight_only_quantized_matmul_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters(workload):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary (copy-calibrated),
    or None when there is none or the kernels changed since it was taken."""
    path = COUNTER_SUMMARY.get(workload)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    sha, traffic = None, None
    with open(os.path.join(ROOT, path)) as f:
        for line in f:
            if line.startswith("kernel source sha256[:16]"):
                sha = line.rsplit(":", 1)[1].strip()
            elif line.startswith("traffic_bytes_per_launch:"):
                traffic = int(line.split(":", 1)[1])
    return traffic if sha == kernel_source_hash() else None


def problems_for(name):
    import synth
    if name == "dense_gemv":
        return [synth.dense_gemv(S=1)], "dense_gemv: int4 W[12288,6144] (codes U{0..15}), scales U[0.002,0.05], x N(0,1), S=1"
    if name.startswith("dense_gemv_s") and name[len("dense_gemv_s"):].isdigit():
        S = int(name[len("dense_gemv_s"):])
        return [synth.dense_gemv(S=S)], ("dense_gemv: int4 W[12288,6144] (codes U{0..15}), scales U[0.002,0.05], "
                                         "x N(0,1), S=%d" % S)
    if name.startswith("moe_decode_s") and name[len("moe_decode_s"):].isdigit():
        S = int(name[len("moe_decode_s"):])
        return synth.moe_decode(S=S), ("moe_decode: 8 experts x int4 {gate,up}[2048,6144] + down[6144,2048], "
                                       "S=%d per expert, all 24 matmuls in one grouped call" % S)
    if name == "moe_decode":
        return synth.moe_decode(), ("moe_decode: 8 experts x int4 {gate,up}[2048,6144] + down[6144,2048], "
                                    "S=1 per expert, all 24 matmuls in one grouped launch")
    if name.startswith("moe_ffn_s") and name[len("moe_ffn_s"):].isdigit():
        S = int(name[len("moe_ffn_s"):])
        return synth.moe_decode(S=S), ("moe_ffn: 8 experts x int4 {gate,up}[2048,6144] -> h = silu(g)*u -> "
                                       "down[6144,2048], S=%d per expert" % S)
    if name in ("moe_ffn", "moe_ffn_pipeline"):
        return synth.moe_decode(), ("moe_ffn: 8 experts x int4 {gate,up}[2048,6144] -> h = silu(g)*u -> "
                                    "down[6144,2048], S=1 per expert, fused gate/up launch + grouped down launch")
    if name.startswith("int2_gemv_s"):
        S = int(name[len("int2_gemv_s"):])
        return [synth.int2_gemv(S=S)], "int2_gemv: int2 W[16384,8192] (codes U{0..3}), scales U[0.01,0.1], S=%d" % S
    if name == "prefill":
        return [synth.prefill(S=512)], "prefill: int8 W[6144,6144] (rint N(0,40) clipped), scales U[0.001,0.01], S=512"
    if name == "dense_gemv_gs128":
        p = synth.dense_gemv(S=1)
        p.gs, p.gscales = 128, synth.group_scales(p, 128, 0.002, 0.05)
        return [p], ("dense_gemv_gs128: int4 W[12288,6144] (codes U{0..15}), one scale per row and group of 128 "
                     "columns U[0.002,0.05], x N(0,1), S=1")
    if name == "dense_gemv_s8_gs128":
        p = synth.dense_gemv(S=8)
        p.gs, p.gscales = 128, synth.group_scales(p, 128, 0.002, 0.05)
        return [p], ("dense_gemv_s8_gs128: int4 W[12288,6144] (codes U{0..15}), one scale per row and group of 128 "
                     "columns U[0.002,0.05], x N(0,1), S=8")
    if name == "prefill_gs128":
        p = synth.prefill(S=512)
        p.gs, p.gscales = 128, synth.group_scales(p, 128, 0.001, 0.01)
        return [p], ("prefill_gs128: int8 W[6144,6144] (rint N(0,40) clipped), one scale per row and group of 128 "
                     "columns U[0.001,0.01], S=512")
    raise ValueError(name)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": 4 * n,
                          "copy_calibration_bytes_written_per_launch": 4 * n, "launches": 10}), flush=True)
        return

    import weight_only_quantized_matmul_amd as wq

    probs, desc = problems_for(args.workload)
    wq.wq_init([0])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup
    grouped = args.workload == "moe_decode" or args.workload.startswith("moe_decode_s")
    ffn = args.workload in ("moe_ffn", "moe_ffn_pipeline") or args.workload.startswith("moe_ffn_s")
    weight_bytes = sum(p.weight_bytes for p in probs)

    def io_bytes(p):  # weights, scales, activations in, results out
        return (p.weight_bytes + 4 * p.O * (p.gscales.shape[1] if getattr(p, "gs", 0) else 1)
                + 4 * p.S * p.I + 4 * p.S * p.O)

    alg_bytes = sum(io_bytes(p) for p in probs)
    if ffn:
        # gate and up read one x and write one h between them; down reads h
        gu_bytes = sum(p.weight_bytes + 4 * p.O for i, p in enumerate(probs) if i % 3 != 2) + sum(
            4 * p.S * p.I + 4 * p.S * p.O for i, p in enumerate(probs) if i % 3 == 0)
        alg_bytes = gu_bytes + sum(io_bytes(p) for i, p in enumerate(probs) if i % 3 == 2)
    alg_flops = sum(2.0 * p.S * p.O * p.I for p in probs)
    compute_bound = args.workload.startswith("prefill")
    n_rot = 1 if compute_bound else max(1, math.ceil(ROTATION_BYTES / weight_bytes))

    # resident weights: n_rot copies of the tensor set
    copies = []
    for _ in range(n_rot):
        copies.append([wq.wq_tensor_upload_gs(None, 0, p.fmt, p.O, p.I, p.gs, p.w, p.gscales) if getattr(p, "gs", 0)
                       else wq.wq_tensor_upload(None, 0, p.fmt, p.O, p.I, p.w, p.scales) for p in probs])
    groups = [wq.wq_grouped_create(c) for c in copies] if grouped else None
    xs = [torch.from_numpy(p.x).to(dev) for p in probs]
    ys = [torch.empty((p.S, p.O), dtype=torch.float32, device=dev) for p in probs]
    if ffn:
        E = len(probs) // 3
        gated = [wq.wq_swiglu_create(c[0::3], c[1::3]) for c in copies]
        downs = [wq.wq_grouped_create(c[2::3]) for c in copies]
        groups = gated + downs
        fx = [xs[3 * e] for e in range(E)]
        fh = [torch.empty((probs[3 * e].S, probs[3 * e].O), dtype=torch.float32, device=dev) for e in range(E)]
        fy = [torch.empty((probs[3 * e].S, probs[3 * e + 2].O), dtype=torch.float32, device=dev)
              for e in range(E)]

    def step(i):
        r = i % n_rot
        if ffn:
            wq.wq_swiglu_ffn_dev(gated[r], downs[r], fx, fh, fy)
        elif grouped:
            wq.wq_grouped_matmul_dev(groups[r], xs, ys)
        else:
            wq.wq_matmul_dev(copies[r][0], xs[0], ys[0])

    def gate_up_only(i):
        wq.wq_swiglu_matmul_dev(gated[i % n_rot], fx, fh)

    stream = torch.cuda.current_stream()
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(K):
                step(i)
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay: instantiation and first-touch costs
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    ev_s = ev0.elapsed_time(ev1) / 1e3
    per_launch = ev_s / K  # average launch duration on the launch stream (s)
    if ffn:
        # the step is two launches (h feeds the down projection): time the
        # dominant one (the fused gate/up launch) in a graph of its own
        g2 = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(g2, stream=side):
            for i in range(K):
                gate_up_only(i)
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g2.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        step_per_launch = per_launch
        per_launch = e0.elapsed_time(e1) / 1e3 / K

    plans = [wq.wq_describe_plan_gs(p.fmt, p.O, p.I, p.S, getattr(p, "gs", 0)) for p in probs]
    tiled = all(pl.startswith("tiled") for pl in plans)
    bf16x3 = tiled and all("mode=bf16x3" in pl for pl in plans)
    if compute_bound or tiled:
        # (int2 at S = 8 also runs on the tiled MFMA path; its value stays GB/s)
        value = alg_flops * K / wall / 1e9 if compute_bound else weight_bytes * K / wall / 1e9
        unit = "GFLOP/s" if compute_bound else "GB/s"
        # The contraction runs on the matrix type of its mode: fp32 MFMA, or
        # bf16 MFMA on three exact bf16 parts of every activation (three
        # matrix products per algorithmic product, so frac <= 1/3 there).
        # The launch time includes the activation split pre-pass.
        roof = {"bound": "mfma", "achieved": alg_flops / per_launch / 1e12,
                "peak": BF16_MFMA_PEAK_TFLOPS if bf16x3 else FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
        if bf16x3:
            roof["issued_mfma_flops_per_launch"] = 3.0 * alg_flops
        if not compute_bound:
            roof["hbm_achieved_gbs"] = alg_bytes / per_launch / 1e9
    elif all(pl.startswith("gemv") for pl in plans) and probs[0].S >= 4 and probs[0].fmt == 3:
        # int2 with S >= 4 activation rows on the register GEMV: S fp32 FMAs
        # per 0.25-byte weight element bind the vector ALUs before HBM (packed
        # fp32 FMAs are not used), so the roofline is the vector FMA rate;
        # HBM rate alongside.
        value = weight_bytes * K / wall / 1e9
        unit = "GB/s"
        roof = {"bound": "alu", "achieved": alg_flops / per_launch / 1e12, "peak": FP32_VALU_FMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "hbm_achieved_gbs": alg_bytes / per_launch / 1e9}
    else:
        value = weight_bytes * K / wall / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": (gu_bytes if ffn else alg_bytes) / per_launch / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        if all(pl.startswith("skinny") for pl in plans):
            # few activation rows on the matrix cores: bounded by the weight
            # bytes; the matrix work (three exact bf16 parts, stacked into the
            # MFMA rows) alongside
            roof["kernel"] = "matrix-core few-rows kernel (S <= 16), one launch"
            roof["mfma_tflops_fp32_equivalent"] = alg_flops / per_launch / 1e12
        if ffn:
            roof["kernel"] = "fused gate/up (paired rows, silu(g)*u epilogue), all experts in one launch"
            roof["step_frac"] = alg_bytes / step_per_launch / 1e9 / HBM_PEAK_GBS
        elif grouped:
            roof["kernel"] = ("grouped GEMV: all 24 matmuls (3 KiB gate/up rows and 1 KiB down rows) "
                              "in one launch; the whole step")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_from_counters(args.workload)

    if roof["bound"] == "hbm" and not args.no_calibration:
        roof["ceiling"] = stream_read_ceiling(torch, wq, weight_bytes, n_rot, min(K, 400), plans[0])

    pipe = None
    if args.workload == "moe_ffn_pipeline":
        pipe = pipeline_modes(torch, wq, gated, downs, probs, n_rot, min(K, 400))
        pipe["graph_replay_us_per_step"] = wall / K * 1e6

    api = None
    if len(probs) == 1 and not getattr(probs[0], "gs", 0):
        api = host_sync_latency(wq, copies[0][0], probs[0].x)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(probs, compute_bound, args.cpu_seconds, ffn=ffn)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16x3 else "f32",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "weight_bytes_per_step": weight_bytes,
            "algorithmic_bytes_per_step": alg_bytes,
            "algorithmic_flops_per_step": alg_flops,
            "weight_copies_rotated": n_rot,
            "launch": "eager" if graph is None else "one HIP graph of K kernel launches",
            "pct_hbm_peak_weight_stream": None if compute_bound else 100.0 * value / HBM_PEAK_GBS,
            "event_us_per_launch": per_launch * 1e6,
            **({"event_us_per_step_two_launches": step_per_launch * 1e6,
                "algorithmic_bytes_gate_up_launch": gu_bytes} if ffn else {}),
            "plan": plans[:3],
            **({"host_sync_api_latency": api} if api else {}),
            **({"pipeline": pipe} if pipe else {}),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)

    if groups:
        for g in groups:
            wq.wq_grouped_free(g)
    for c in copies:
        for t in c:
            wq.wq_tensor_free(t)


def stream_read_ceiling(torch, wq, nbytes, n_rot, K, plan):
    """Practical HBM read ceiling for this step's weight bytes: a plain 128-bit non-temporal
    stream read of the same byte count, over the same number of rotated copies, for a few
    launch shapes (waves x 1 KiB loads in flight per wave), each timed over K launches in
    one HIP graph like the workload. Returns the best rate and every shape's rate (GB/s)."""
    dev = torch.device("cuda:0")
    n16 = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n16 // 4, dtype=torch.int32, device=dev) for _ in range(n_rot)]
    # whole chunk in flight at once (one round trip per wave) at 1, 2, 4 and 8 waves per
    # SIMD, plus the shape of a 4-row ring of 3 KiB rows (12 loads of 1 KiB)
    kib = -(-nbytes // 1024)
    shapes = [(1024, 12)]
    for waves in (1024, 2048, 4096, 8192):
        need = -(-kib // waves)
        loads = next((L for L in (1, 2, 4, 5, 8, 9, 12, 16, 18, 24, 36) if L >= need), 36)
        shapes.append((waves, loads))
    out = torch.empty(64 * max(w for w, _ in shapes), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rates = {}
    for waves, loads in shapes:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(K):
                wq.wq_stream_read_dev(bufs[i % n_rot], waves, loads, out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        rates["%dx%d" % (waves, loads)] = {"us": round(us, 3), "gbs": round(nbytes / us / 1e3, 1)}
        del g
    best = max(rates.items(), key=lambda kv: kv[1]["gbs"])
    del bufs
    return {"kernel": "stream read, 128-bit non-temporal loads, same byte count and rotation",
            "bytes_per_launch": nbytes, "best_shape": best[0], "best_gbs": best[1]["gbs"],
            "best_us": best[1]["us"], "shapes_waves_x_loads": rates}


def pipeline_modes(torch, wq, gated, downs, probs, n_rot, K):
    """Per-step time (us) of the 8-expert feed-forward in different host/device arrangements.

    Eager modes are launched from Python one call at a time; graph modes
    capture the same K steps (copies, kernels, cross-stream event waits) into
    one HIP graph and replay it."""
    dev = torch.device("cuda:0")
    E = len(probs) // 3
    S, I, F, Od = probs[0].S, probs[0].I, probs[0].O, probs[2].O
    gen = torch.Generator().manual_seed(20261202)
    x_host = torch.empty((K, E, S, I), dtype=torch.float32, pin_memory=True)
    x_host.copy_(torch.randn((K, E, S, I), generator=gen))
    y_host = torch.empty((K, E, S, Od), dtype=torch.float32, pin_memory=True)
    xd = [torch.zeros((E, S, I), device=dev) for _ in range(2)]
    hd = [torch.empty((E, S, F), device=dev) for _ in range(2)]
    yd = [torch.empty((E, S, Od), device=dev) for _ in range(2)]
    cin, cout = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    ev_in = [torch.cuda.Event() for _ in range(2)]
    ev_done = [torch.cuda.Event() for _ in range(2)]
    ev_out = [torch.cuda.Event() for _ in range(2)]

    def ffn(t, b, comp):
        wq.wq_swiglu_ffn_dev(gated[t % n_rot], downs[t % n_rot], list(xd[b]), list(hd[b]), list(yd[b]),
                             stream=comp)

    def device_resident(comp):
        for t in range(K):
            ffn(t, 0, comp)

    def host_io_serialised(comp):
        for t in range(K):
            xd[0].copy_(x_host[t], non_blocking=True)
            ffn(t, 0, comp)
            y_host[t].copy_(yd[0], non_blocking=True)

    def host_io_overlapped(comp):
        # step t uses slot t % 2: x of step t + 1 goes up (stream cin) and y
        # of step t - 1 comes down (stream cout) while step t computes
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
            ffn(t, b, comp)
            ev_done[b].record(comp)
            with torch.cuda.stream(cout):
                cout.wait_event(ev_done[b])
                y_host[t].copy_(yd[b], non_blocking=True)
                ev_out[b].record(cout)
        comp.wait_event(ev_out[(K - 1) % 2])  # join the output stream

    def eager(body, sync_each=False):
        comp = torch.cuda.current_stream()
        if not sync_each:
            return lambda: body(comp)

        def run():
            for t in range(K):
                xd[0].copy_(x_host[t], non_blocking=True)
                ffn(t, 0, comp)
                y_host[t].copy_(yd[0], non_blocking=True)
                torch.cuda.synchronize()
        return run

    def graphed(body):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            body(side)
        torch.cuda.synchronize()
        return g.replay

    def timed(run):
        run()  # warm-up pass
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K * 1e6

    out = {}
    for name, run in (("eager_device_resident", eager(device_resident)),
                      ("eager_host_io_serialised", eager(host_io_serialised)),
                      ("eager_host_io_sync_each_step", eager(None, sync_each=True)),
                      ("eager_host_io_overlapped", eager(host_io_overlapped)),
                      ("graph_device_resident", graphed(device_resident)),
                      ("graph_host_io_serialised", graphed(host_io_serialised)),
                      ("graph_host_io_overlapped", graphed(host_io_overlapped))):
        y_host.zero_()
        out[name + "_us_per_step"] = timed(run)
        if "host_io" in name:  # the outputs that came back equal eager ones from the same inputs
            ok = True
            for t in sorted({0, 1, K // 2, K - 1}):
                xd[0].copy_(x_host[t])
                ffn(t, 0, torch.cuda.current_stream())
                torch.cuda.synchronize()
                ok = ok and torch.equal(yd[0].cpu(), y_host[t])
            out[name + "_outputs_checked"] = bool(ok)
    out["steps"] = K
    out["host_bytes_per_step"] = 4 * E * S * (I + Od)
    return out


def host_cpu():
    """(nproc, cores this process may use, CPU model name) of the host."""
    nproc = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = nproc
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return nproc, usable, model


def cpu_baseline(probs, compute_bound, seconds, ffn=False):
    """The CPU oracle as it stands, on this host: one warm-up run, then the median of five
    timed runs, on one thread and on every core the process may use (capped by
    OMP_NUM_THREADS when set: the machine's CPU share). A run is a fixed number of passes over
    a bounded sample of the workload, sized so that the whole measurement takes about
    `seconds` (single-thread runs dominate)."""
    import statistics

    import oracle
    nproc, usable, model = host_cpu()
    all_threads = usable
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        all_threads = max(1, min(all_threads, int(os.environ["OMP_NUM_THREADS"])))

    if ffn:  # the oracle's gate, up, silu_mul, down chain per expert
        E = len(probs) // 3
        unit_work = sum(p.weight_bytes for p in probs)

        def one_pass(threads):
            for e in range(E):
                gp, up, dp = probs[3 * e:3 * e + 3]
                g, _ = oracle.matmul(gp.fmt, gp.w, gp.scales, gp.x, threads=threads, want_bound=False)
                u, _ = oracle.matmul(up.fmt, up.w, up.scales, gp.x, threads=threads, want_bound=False)
                h = oracle.silu_mul(g, u)
                oracle.matmul(dp.fmt, dp.w, dp.scales, h, threads=threads, want_bound=False)
        desc = "the 8-expert gate/up/silu/down chain, S=1"
    else:
        # bounded sample: whole weight matrices, at most 16 activation rows of each
        sample = [(p, p.x[:min(p.S, 16)]) for p in probs]
        unit_work = sum((2.0 * x.shape[0] * p.O * p.I) if compute_bound else p.weight_bytes for p, x in sample)

        def one_pass(threads):
            for p, x in sample:
                if getattr(p, "gs", 0):
                    oracle.matmul_gs(p.fmt, p.w, p.gscales, p.gs, x, threads=threads, want_bound=False)
                else:
                    oracle.matmul(p.fmt, p.w, p.scales, x, threads=threads, want_bound=False)
        desc = "%s with S<=16 activation rows" % "+".join(sorted(set(p.name.split("_")[0] for p, _ in sample)))[:60]

    def timed(threads, passes):
        t0 = time.perf_counter()
        for _ in range(passes):
            one_pass(threads)
        return time.perf_counter() - t0

    # size the runs: 6 single-thread runs take about `seconds`
    probe = timed(1, 1)
    passes = max(1, int(seconds / 6.0 / max(probe, 1e-6)))
    out = {}
    for label, threads in (("one_thread", 1), ("all_cores", all_threads)):
        timed(threads, passes)  # warm-up
        runs = [timed(threads, passes) for _ in range(5)]
        med = statistics.median(runs)
        out[label] = {"threads": threads, "value": unit_work * passes / med / 1e9,
                      "median_s": med, "runs_s": [round(r, 4) for r in runs]}
    unit = "GFLOP/s" if compute_bound else "GB/s"
    return {"value": out["all_cores"]["value"], "unit": unit, "cores": all_threads, "kind": "oracle",
            "sample": "%d pass(es) per run over %s; median of 5 runs after 1 warm-up" % (passes, desc),
            "one_thread_value": out["one_thread"]["value"], "nproc": nproc, "usable_cores": usable,
            "cpu_model": model, "runs": out}


def host_sync_latency(wq, t, x, calls=200):
    """Latency of the synchronous host-pointer call (blocking H2D of x, launch, D2H of y,
    stream synchronisation): median and spread over `calls` calls after 20 warm-up calls."""
    import statistics
    for _ in range(20):
        wq.wq_matmul_t(t, x)
    lat = []
    for _ in range(calls):
        t0 = time.perf_counter()
        wq.wq_matmul_t(t, x)
        lat.append((time.perf_counter() - t0) * 1e6)
    lat.sort()
    return {"median_us": statistics.median(lat), "p10_us": lat[len(lat) // 10], "p90_us": lat[9 * len(lat) // 10],
            "calls": calls, "host_bytes_in": int(x.nbytes), "host_bytes_out": int(4 * x.shape[0] * t.O)}


if __name__ == "__main__":
    main()
