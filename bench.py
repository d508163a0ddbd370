#!/usr/bin/env python3
"""Throughput of the fused NHWC int8 convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one fconv_plan_run of the whole layer (implicit-GEMM conv with the
fused scale / side-input / bias / ReLU / requantise epilogue) over the full
synthetic batch, inputs already resident in HBM, filter packed once per plan
(as inference with fixed weights does).  W untimed steps, then exactly K
timed steps bracketed by torch.cuda.synchronize(); prints ONE JSON line.

The K timed steps are issued one of two ways, chosen by K alone: for K >= 64,
K fconv_plan_run calls captured into one HIP graph and replayed once (the
graph removes the per-call host launch cost, but its submission costs a fixed
15-20 us that only many launches amortize); for smaller K, the K calls issued
eagerly, one launch each (the first kernel starts at once and the host's
later launches overlap the kernels before them).  Every step runs the full
kernel either way, and both ways are measured and reported; the other way's
figures sit beside the headline ("graph", "eager"), and so does a cold run
with the 256 MB last-level cache flushed (1 GiB written) before each step.

value  = 2*N*Ho*Wo*K*R*S*C * K_steps / wall seconds of the K timed steps, TOPS.
roofline: the conv kernel's algorithmic bytes (x + filter + side + y + bias,
each once) or operations per launch / its average launch duration from HIP
events recorded on the launch stream around the timed region.
cpu_baseline: the CPU oracle (direct loops + epilogue) timed on the host
cores on the same workload.
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused int8 conv TOPS (2·N·Ho·Wo·K·R·S·C/t) and % of MFMA peak, 1 GPU"
PEAK_HBM_GBS = 8000.0
PEAK_TOPS = {"int8": 5000.0, "bf16": 2500.0, "fp32": 157.3}  # dense MFMA
KERNEL_SOURCES = [os.path.join(ROOT, "convolution_implicit_gemm_nhwc_amd", "csrc", f)
                  for f in ("conv.hip", "plan.cpp", "plan.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _code_only(text: str) -> str:
    """C/C++ source without its comments and blank lines: what the compiler
    turns into kernels (a comment edit leaves the counters valid)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


# Steps from which the timed K steps run as one HIP graph replay (below: eager
# launches).  Measured on one MI355X (wall us per step, graph / eager): the
# int8 3x3 layer 11.05 / 10.31 at K = 20 and 8.55 / 8.89 at K = 200; the bf16
# 3x3 layer 25.0 / 24.15 and 22.57 / 24.26.
GRAPH_MIN_STEPS = 64


def launch_note(use_graph: bool) -> str:
    how = ("the K steps as one hip graph, replayed once" if use_graph else
           "the K steps launched eagerly, one launch each (K < %d)" % GRAPH_MIN_STEPS)
    return (how + " (value, ms_per_step: host wall clock with a synchronize on both sides; "
            "graph / eager: both ways' figures, event_us_per_step from HIP events around "
            "them); roofline.kernel_avg_us: HIP events around a later replay of the graph "
            "queued behind others, i.e. the launches' own GPU time back to back")


def kernel_source_hash(sources=None) -> str:
    """Hash of the code of the kernel sources the counters were taken on (the
    forward kernels' by default; an entry may name its own files)."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if sources is None else [os.path.join(ROOT, x) for x in sources]):
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(L, per_channel_scale=False) -> int:
    """Each tensor once: x, filter, side input, y, per-channel vectors."""
    esize = {"int8": 1, "bf16": 2, "fp32": 4}[L.dtype]
    x = L.N * L.H * L.W * L.C * esize
    w = L.R * L.S * L.C * L.K * esize
    y = L.N * L.Ho * L.Wo * L.K * esize
    side = L.N * L.Ho * L.Wo * L.K if L.has_side else 0
    nvec = 1 + (4 if L.dtype != "int8" and 4 in L.ops else 0) + (1 if per_channel_scale else 0)
    return x + w + y + side + 4 * L.K * nvec


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel") != kernel or \
            e.get("source_hash") != kernel_source_hash(e.get("sources")):
        return None
    return e.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _timed_oracle(L, x, w, inp, cis, order, seconds, form):
    """Repeat the oracle's fused conv on (x, w) for about `seconds`; returns
    the last output and the rate in TOPS of the layer's arithmetic."""
    import oracle
    n = x.shape[0]
    side = inp.side[:n] if inp.side is not None else None
    reps, t0 = 0, time.perf_counter()
    while True:
        acc = oracle.conv_acc(x, w, L.stride, L.padding, form=form)
        y = oracle.epilogue_i8(acc, cis, inp.bias, side, L.side_input_scale, L.relu, order)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return y, reps, dt, L.ops_count() * n / L.N * reps / dt / 1e12


def cpu_baseline(L, inp, seconds: float, cis=None, order=8):
    """The CPU oracle timed on the host: the direct seven-loop form on all
    cores (the headline baseline, checked against the GPU's output), on one
    core (a bounded sample of the batch), and the im2col + GEMM form on all
    cores."""
    import oracle
    cis = L.conv_input_scale if cis is None else cis
    cores = oracle.num_threads()  # the host's OpenMP default (all the cores it grants)
    y, reps, dt, tops = _timed_oracle(L, inp.x, inp.w, inp, cis, order, seconds, "direct")
    out = dict(value=round(tops, 6), unit="TOPS", cores=cores, kind="oracle",
               sample="full %s batch (N=%d), %d repetition(s) in %.1f s: direct 7-loop conv + "
                      "int8 epilogue, OpenMP over (n, ho)" % (L.name, L.N, reps, dt),
               cpu_model=cpu_model())
    # One core, on the first image(s) of the batch (a bounded sample).
    n1 = max(1, min(L.N, int(2e9 // max(1, L.ops_count() // L.N))))
    oracle.set_num_threads(1)
    _, r1, d1, t1 = _timed_oracle(L, inp.x[:n1], inp.w, inp, cis, order, seconds / 2, "direct")
    out["single_thread"] = dict(value=round(t1, 6), unit="TOPS", cores=1,
                                sample="first %d image(s), %d repetition(s) in %.1f s: direct form"
                                       % (n1, r1, d1))
    # The im2col + GEMM form, all cores, on the same sample size.
    oracle.set_num_threads(cores)
    _, r2, d2, t2 = _timed_oracle(L, inp.x[:n1], inp.w, inp, cis, order, seconds / 2, "im2col")
    out["im2col"] = dict(value=round(t2, 6), unit="TOPS", cores=oracle.num_threads(),
                         sample="first %d image(s), %d repetition(s) in %.1f s: per-image "
                                "im2col patch matrix x [R*S*C, K] filter" % (n1, r2, d2))
    return y, out


def copy_probe(nbytes: int, steps: int, warmup: int):
    """Plain device copy of nbytes (read nbytes, write nbytes): the known-size
    kernel whose FETCH_SIZE / WRITE_SIZE calibrate the conv kernel's counters,
    and a practical ceiling for streaming bandwidth on this GPU."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    a.random_()
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        b.copy_(a)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    print(json.dumps({"copy_bytes": a.numel() * 4, "us_per_copy": round(us, 3),
                      "GBps_read_plus_write": round(2 * a.numel() * 4 / (us * 1e-6) / 1e9, 1)}),
          flush=True)


def gated_graph_ms(graph, gstream, steps: int) -> float:
    """GPU time per launch of one replay of `graph` (`steps` launches),
    queued behind other replays of the same graph (about 200 launches in
    all): the host has submitted it before the first event is stamped, so
    the events bracket the launches back to back on a busy GPU, not the
    host-side launch of the graph, which a replay timed on its own also
    includes (~1 us per step at 20 steps)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(gstream):
        for _ in range(max(1, 200 // steps)):
            graph.replay()
        e0.record(gstream)
        graph.replay()
        e1.record(gstream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def wgrad_cpu_baseline(L, inp, seconds: float):
    """The oracle's weight gradient on a prefix of the batch (one image, then
    more while the budget lasts), as FLOP/s of the same formula."""
    import oracle
    n_img = 1
    reps, flops, t0 = 0, 0, time.perf_counter()
    ref = None
    while True:
        ref = oracle.wgrad(inp.x[:n_img], inp.dy[:n_img], L.R, L.S, L.stride, L.padding)
        reps += 1
        flops += L.ops_count() // L.N * n_img
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    # The oracle's parallel loop runs over the R*S filter taps.
    return ref, n_img, dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s",
                            cores=min(oracle.num_threads(), L.R * L.S), kind="oracle",
                            sample="first image of the %s batch, %d repetition(s) in %.1f s: "
                                   "direct loops in double, OpenMP over (r, s)"
                                   % (L.name, reps, dt))


def bench_wgrad(args):
    """Weight gradient: dw of the layer from x and dy, fp32 dW (bf16 inputs)."""
    import numpy as np
    import torch

    import convolution_implicit_gemm_nhwc_amd as fc
    import workloads as wl

    L = wl.WGRAD_LAYERS[args.workload]
    dev = torch.device("cuda:0")
    inp = wl.make_wgrad_inputs(L)
    plan = fc.WgradPlan(L.N, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                        out_fp32=True)

    def put(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x, dy = put(inp.x), put(inp.dy)
    dw = torch.empty(plan.dw_shape, dtype=torch.float32, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(h):
        st = plan.run_raw(x, dy, dw, ws, stream=h)
        if st != 0:
            raise fc.FconvError(st, "fconv_wgrad_plan_run")

    for _ in range(args.warmup):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step(stream.cuda_stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    eager_ms = ev0.elapsed_time(ev1) / args.steps

    gstream = torch.cuda.Stream()
    gstream.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(graph, stream=gstream):
            for _ in range(args.steps):
                step(gstream.cuda_stream)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(gstream)
    with torch.cuda.stream(gstream):
        graph.replay()
    g1.record(gstream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_event_ms = g0.elapsed_time(g1) / args.steps
    step_ms = gated_graph_ms(graph, gstream, args.steps)

    ops = L.ops_count()
    esize = 2 if L.dtype == "bf16" else 4
    alg_bytes = (L.N * L.H * L.W * L.C + L.N * L.Ho * L.Wo * L.K) * esize + \
        L.R * L.S * L.C * L.K * 4
    use_graph = args.steps >= GRAPH_MIN_STEPS
    wall_timed = wall if use_graph else wall_eager
    value = ops * args.steps / wall_timed / 1e12
    peak = PEAK_TOPS[L.dtype]
    achieved = ops / (step_ms * 1e-3) / 1e12
    kernels = plan.kernel_name + ("+wgrad_reduce" if plan.workspace_bytes else "")
    out = {
        "metric": "conv weight-gradient TFLOP/s (2*N*Ho*Wo*K*R*S*C/t), 1 GPU",
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_timed / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16 (fp32 accumulate, fp32 dW)", "fp32": "fp32"}[L.dtype],
        "data": "synthetic",
        "config": {"workload": L.name, "layer": L.description, "N": L.N, "H": L.H, "W": L.W,
                   "C": L.C, "K": L.K, "R": L.R, "S": L.S, "stride": L.stride,
                   "padding": L.padding, "kernel": kernels,
                   "pixel_ranges": plan.workspace_bytes // (16 * ((L.R * L.S * L.C * L.K + 3)
                                                                 // 4)) or 1},
        "launch": launch_note(use_graph),
        "pct_of_mfma_peak": round(100.0 * value / peak, 3),
        "graph_event_us_per_step": round(graph_event_ms * 1e3, 3),
        "graph": {"value": round(ops * args.steps / wall / 1e12, 4),
                  "ms_per_step": round(wall / args.steps * 1e3, 6),
                  "event_us_per_step": round(graph_event_ms * 1e3, 3)},
        "eager": {"value": round(ops * args.steps / wall_eager / 1e12, 4),
                  "ms_per_step": round(wall_eager / args.steps * 1e3, 6),
                  "event_us_per_step": round(eager_ms * 1e3, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(L.name, kernels),
                     "kernel": kernels, "kernel_avg_us": round(step_ms * 1e3, 3),
                     "note": "one step = the main kernel and the fixed-order sum of its "
                             "pixel ranges, timed together; traffic is the step's (both "
                             "kernels, the partial sums' round trip included)",
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        ref, n_img, cb = wgrad_cpu_baseline(L, inp, args.cpu_seconds)
        # The sample's own check: the GPU on the same image prefix.
        g = fc.WgradPlan(n_img, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                         out_fp32=True)
        dw1 = g(x[:n_img].contiguous(), dy[:n_img].contiguous())
        torch.cuda.synchronize()
        got = dw1.cpu().numpy().astype(np.float64)
        cb["sample_normwise_error_vs_gpu"] = float(np.max(np.abs(got - ref)) /
                                                   max(np.max(np.abs(ref)), 1e-300))
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="resnet_3x3_int8")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-channel-scale", action="store_true",
                    help="int8: one conv_input_scale per output channel (the layer's scale "
                         "times a seeded factor in [0.5, 2))")
    ap.add_argument("--cudnn7-order", action="store_true",
                    help="int8: the cuDNN 7 epilogue order (fused scale and bias)")
    ap.add_argument("--activation", default=None, metavar="NAME[:ALPHA[:BETA]]",
                    help="bf16/fp32: replace the layer's ReLU by leaky_relu, clipped_relu or "
                         "clamp with these arguments")
    ap.add_argument("--autotune", action="store_true",
                    help="time every kernel configuration for the layer first and run the "
                         "fastest (fconv_plan_autotune)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="instead of the conv, time a plain device-to-device copy of "
                         "BYTES bytes (the reference kernel for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the fused convolution is batch-parallel "
              "with no cross-GPU exchange, and this build runs on a single MI355X. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps, args.warmup)
        return

    import convolution_implicit_gemm_nhwc_amd as fc
    import workloads as wl

    if args.workload in wl.WGRAD_LAYERS:
        bench_wgrad(args)
        return
    L = wl.LAYERS[args.workload]
    if (args.per_channel_scale or args.cudnn7_order) and L.dtype != "int8":
        print("--per-channel-scale and --cudnn7-order apply to int8 layers", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    inp = wl.make_inputs(L)
    names = {wl.OP_SCALE: "scale", wl.OP_SIDE: "side", wl.OP_BIAS: "bias", wl.OP_BN: "bn",
             wl.OP_RELU: "relu"}
    opnames = [names[o] for o in L.ops]
    act_alpha = act_beta = 0.0
    if args.activation:
        if L.dtype == "int8":
            print("--activation applies to bf16/fp32 layers", file=sys.stderr)
            sys.exit(2)
        parts = args.activation.split(":")
        act_alpha = float(parts[1]) if len(parts) > 1 else 0.0
        act_beta = float(parts[2]) if len(parts) > 2 else 0.0
        opnames = [o for o in opnames if o != "relu"] + [parts[0]]
    plan = fc.Plan(L.N, L.H, L.W, L.C, L.K, L.R, L.S, L.stride, L.padding, L.dtype,
                   ops=opnames, cudnn7_order=args.cudnn7_order)
    order = 7 if args.cudnn7_order else 8
    cis_host = L.conv_input_scale
    if args.per_channel_scale:
        rng = np.random.default_rng(1000 + L.seed)
        cis_host = (np.float32(L.conv_input_scale) *
                    rng.uniform(0.5, 2.0, size=L.K)).astype(np.float32)

    def put(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x, w, bias, side = put(inp.x), put(inp.w), put(inp.bias), put(inp.side)
    cis = put(cis_host) if args.per_channel_scale else L.conv_input_scale
    bn = None
    if inp.bn is not None:
        bn = {k: put(np.asarray(inp.bn[k], np.float32)) for k in ("gamma", "beta", "mean", "var")}
        bn["eps"] = float(inp.bn["eps"])
    tdt = {"int8": torch.int8, "bf16": torch.bfloat16, "fp32": torch.float32}[L.dtype]
    y = torch.empty(plan.out_shape, dtype=tdt, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    plan.pack_filter(w, ws, stream)
    run_args = plan.make_args(x, w, y, ws, bias=bias, side=side,
                              conv_input_scale=cis,
                              side_input_scale=L.side_input_scale, bn=bn, prepacked=True,
                              activ_alpha=act_alpha, activ_beta=act_beta)
    full_args = plan.make_args(x, w, y, ws, bias=bias, side=side,
                               conv_input_scale=cis,
                               side_input_scale=L.side_input_scale, bn=bn, prepacked=False,
                               activ_alpha=act_alpha, activ_beta=act_beta)
    h = stream.cuda_stream
    heuristic_kernel = plan.kernel_name
    if args.autotune:
        fc.autotune_cache_clear()
        plan.autotune(x, w, y, ws, repeats=20, stream=stream, bias=bias, side=side,
                      conv_input_scale=cis, side_input_scale=L.side_input_scale, bn=bn,
                      prepacked=True, activ_alpha=act_alpha, activ_beta=act_beta)

    def step(a=run_args):
        st = plan.run_args(a, h)
        if st != 0:
            raise fc.FconvError(st, "fconv_plan_run")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Eager: K calls, one launch each.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    eager_ms = ev0.elapsed_time(ev1) / args.steps

    # Graph: the same K calls captured once, replayed once (timed).
    gstream = torch.cuda.Stream()
    gstream.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(graph, stream=gstream):
            for _ in range(args.steps):
                st = plan.run_args(run_args, gstream.cuda_stream)
                if st != 0:
                    raise fc.FconvError(st, "fconv_plan_run (capture)")
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(gstream)
    with torch.cuda.stream(gstream):
        graph.replay()
    g1.record(gstream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_event_ms = g0.elapsed_time(g1) / args.steps
    kernel_ms = gated_graph_ms(graph, gstream, args.steps)
    y_gpu = y.cpu()

    # Cold: last-level cache flushed before each singly timed step.
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    cold = []
    for i in range(min(args.steps, 20)):
        flush.fill_(i)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        step()
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    del flush
    cold_ms = sorted(cold)[len(cold) // 2]

    # End to end including the per-call filter repack (not the headline).
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step(full_args)
    torch.cuda.synchronize()
    wall_full = time.perf_counter() - t2

    ops = L.ops_count()
    use_graph = args.steps >= GRAPH_MIN_STEPS
    wall_timed = wall if use_graph else wall_eager
    value = ops * args.steps / wall_timed / 1e12
    alg_bytes = algorithmic_bytes(L, args.per_channel_scale)
    # The committed counters were taken with the default epilogue.
    traffic = (None if args.per_channel_scale or args.cudnn7_order or args.activation
               or args.autotune else measured_traffic(L.name, plan.kernel_name))
    # Bound: the roofline the layer meets first (ridge = peak ops / peak bytes).
    ridge = PEAK_TOPS[L.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ops / alg_bytes <= ridge:
        roof = {"bound": "hbm", "achieved": alg_bytes / (kernel_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": ops / (kernel_ms * 1e-3) / 1e12,
                "peak": PEAK_TOPS[L.dtype], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["achieved"] = round(roof["achieved"], 2)
    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_timed / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8": "int8 (int32 accumulate)", "bf16": "bf16 (fp32 accumulate)",
                  "fp32": "fp32"}[L.dtype],
        "data": "synthetic",
        "config": {"workload": L.name, "layer": L.description, "N": L.N, "H": L.H, "W": L.W,
                   "C": L.C, "K": L.K, "R": L.R, "S": L.S, "stride": L.stride,
                   "padding": L.padding, "filter": "prepacked once per plan",
                   "kernel": plan.kernel_name,
                   "kernel_choice": "autotuned (heuristic: %s)" % heuristic_kernel
                   if args.autotune else "heuristic"},
        "epilogue": ("cuDNN %d order, %s conv_input_scale" %
                     (order, "per-channel" if args.per_channel_scale else "scalar")
                     if L.dtype == "int8" else "bias, batch norm, " +
                     (args.activation or "relu")),
        "launch": launch_note(use_graph),
        "pct_of_mfma_peak": round(100.0 * value / PEAK_TOPS[L.dtype], 3),
        "graph_event_us_per_step": round(graph_event_ms * 1e3, 3),
        "graph": {"value": round(ops * args.steps / wall / 1e12, 4),
                  "ms_per_step": round(wall / args.steps * 1e3, 6),
                  "event_us_per_step": round(graph_event_ms * 1e3, 3)},
        "eager": {"value": round(ops * args.steps / wall_eager / 1e12, 4),
                  "ms_per_step": round(wall_eager / args.steps * 1e3, 6),
                  "event_us_per_step": round(eager_ms * 1e3, 3)},
        "cold_llc": {"us_per_step": round(cold_ms * 1e3, 3),
                     "value": round(ops / (cold_ms * 1e-3) / 1e12, 4),
                     "note": "1 GiB written before each step; median of %d" % len(cold)},
        "tops_with_filter_repack_each_step": round(ops * args.steps / wall_full / 1e12, 4),
        "roofline": dict(roof, traffic=traffic, kernel=plan.kernel_name,
                         kernel_avg_us=round(kernel_ms * 1e3, 3),
                         algorithmic_bytes_per_launch=alg_bytes),
    }
    if not args.no_cpu_baseline and L.dtype == "int8":
        y_ref, cb = cpu_baseline(L, inp, args.cpu_seconds, cis_host, order)
        cb["sample_matches_gpu"] = bool(np.array_equal(y_ref, y_gpu.numpy()))
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
