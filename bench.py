"""Benchmark: SVDQuant W4A4 linear on one MI355X.

Step = one forward of the DiT attention QKV projection as a W4A4 linear:
svdq_quantize_act (smoothing + rank-32 down-projection + INT4 g64 activation
quantisation) followed by svdq_gemm_w4a4 (group GEMM + low-rank up-projection
+ bias, bf16 out), M=4096 tokens, K=3072, N=9216, rank 32. `value` is the
effective TOPS of that linear, 2*M*N*K / step time.

Protocol: the first step is timed alone (first_run); the shader clock is read
idle, after the timed steps and after each GEMM repetition set; one second of
steps runs before anything is timed (clock and power ramp); then the K timed
steps (no events inside them), the same K steps with HIP events around each
GEMM (the GEMM's duration inside the step: the roofline figure), the GEMM alone (5 x 50 launches hot, and over 4 rotated operand sets),
the activation kernel over 12 rotated copies of X, a 256 MiB device copy.

In the same run (separate timed loops, reported under "extra"): the AWQ W4A16
adaLN GEMV (4 x 3072 -> 18432, weights rotated through more buffers than the
256 MB Infinity Cache holds, so every launch reads HBM; a read-only probe of
the same bytes beside it), the MLP pair (fc1 3072 -> 12288 with the GELU
epilogue, then fc2 12288 -> 3072, 4608 tokens) unfused and with fc2's
activation pass fused into fc1 (eager and as one HIP graph), the MXFP4
transformer block, the GPU offline quantiser on the QKV weight, and the CPU
oracle (one and all host threads).

Inputs are seeded synthetic tensors resident in HBM before timing starts:
activations with the workload's outlier channels; packed weights are uniform
random sign-magnitude codes with fp16 scales of the prepared layer's
magnitude (kernel time does not depend on the values; parity against the
oracle-prepared layers is the tests' job).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP6_TFLOPS = 10100.0     # MI355X dense FP6 MFMA: the instruction the INT4 GEMM runs on
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense FP4 MFMA (the MXFP4 GEMM)
PEAK_INT8_TOPS = 5000.0       # MI355X dense INT8 MFMA: the integer peak INT4 x INT4 is quoted against
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# HBM traffic of one GEMM launch on the QKV shape, from two rocprofv3 counter
# passes over this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by the factor that makes the same counter read the known size of
# the device copies this script also runs (a copy reads what it writes, and
# WRITE_SIZE counts the written bytes exactly).  The figures hold only for the
# kernel sources they were taken on (their sha256 below); otherwise the
# traffic is reported as null.
GEMM_TRAFFIC = {
    "source_sha256": "1ea68aef412184ed85ff3f62452ab3ef0c8a6a3872eee4c84e684c0e7d328026",
    "fetch_kib": 64083.6, "write_kib": 73728.0,          # QKV GEMM, mean of 3236 / 3616 dispatches
    "fetch_factor": 128134.0 / 64078.7,                   # device copies: bytes written / FETCH_SIZE
    "write_factor": 1.0,                                  # WRITE_SIZE reads the bytes written
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def synth_linear(M, K, N, rank, seed, device):
    """Seeded synthetic operands of one W4A4 linear (layouts of include/svdq.h)."""
    import numpy as np
    import torch

    import synth
    from bit_quantized_diffusion_svdq_amd import pack_l1
    cfg = synth.LayerConfig("bench", M=M, K=K, N=N, rank=rank, n_outliers=max(1, round(0.01 * K)),
                            outlier_factor=30.0, seed=seed)
    li = synth.make_layer(cfg)
    rng = np.random.default_rng(seed + 1)
    g = torch.Generator().manual_seed(seed + 2)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    ops = dict(
        x=bf16(li.x),
        inv_lambda=torch.from_numpy(rng.uniform(0.05, 1.0, K).astype(np.float32)).to(device),
        l1t=pack_l1((torch.randn((K, rank), generator=g) * 0.05).to(torch.bfloat16)).to(device),
        l2t=(torch.randn((N, rank), generator=g) * 0.1).to(torch.bfloat16).to(device),
        qw=torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8).to(device),
        sw=(torch.rand(((K // 64 + 3) // 4, N, 4), generator=g) * 0.02 + 0.01).to(torch.float16).to(device),
        bias=bf16(li.bias),
    )
    return ops


def run_linear(lib, ops, rank, act="none", y=None):
    qx, sx, xl1 = lib.quantize_act(ops["x"], ops["inv_lambda"], ops["l1t"], rank)
    return lib.w4a4_linear(qx, sx, xl1, ops["qw"], ops["sw"], ops["l2t"], ops["bias"], rank,
                           act=act, y=y)


def time_events(fn, iters):
    """Average duration (ms) of fn() over iters launches, by HIP events on the
    current stream (the stream the kernels are launched on)."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def time_reps(fn, per_rep, reps=5, clock=None):
    """reps repetitions of per_rep back-to-back launches of fn(), each timed by
    HIP events on the launch stream; returns per-launch ms of every repetition
    (and the shader clock read right after each one, when `clock` is given)."""
    out, mhz = [], []
    for _ in range(reps):
        out.append(time_events(fn, per_rep))
        if clock is not None:
            mhz.append(clock())
    return out, mhz


def summary_us(ms_list):
    import statistics
    return {"median_us": round(statistics.median(ms_list) * 1e3, 2), "min_us": round(min(ms_list) * 1e3, 2),
            "reps_us": [round(x * 1e3, 2) for x in ms_list]}


def time_graph(fn, per_graph, replays=20):
    """Average duration (ms) of one fn() when per_graph launches are captured in
    a HIP graph and replayed back to back (no host launch gaps between them),
    timed by HIP events on the replay stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()                     # warm: any first-use host set-up happens outside capture
        with torch.cuda.graph(g, stream=st):
            for _ in range(per_graph):
                fn()
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / (replays * per_graph)


def make_clock(lib, dev):
    """Shader clock (MHz) right now: the probe counts shader-clock ticks
    against the 100 MHz real-time counter over a ~50 us busy loop."""
    import torch
    ticks = torch.zeros(2, dtype=torch.int64, device=dev)

    def clock():
        lib.svdq_probe_clock(ticks, 6000)
        t = ticks.cpu().tolist()
        return round(100.0 * t[0] / max(t[1], 1), 1)
    return clock


def settle(fn, seconds):
    """Run fn() back to back for `seconds` of wall time so the chip reaches the
    clock it holds under sustained load; returns the number of calls."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def gemm_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_w4a4.hip", "common.h"):
        with open(os.path.join(ROOT, "bit_quantized_diffusion_svdq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm_traffic_bytes():
    """HBM bytes per GEMM launch from the recorded counter passes, or None when
    the kernel sources have changed since they were taken."""
    t = GEMM_TRAFFIC
    if t is None or t["source_sha256"] != gemm_source_digest():
        return None
    return int(round(1024 * (t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"])))


def offline_quantize_timing(lib, dev, reps=5, fmt="int4"):
    """The GPU offline quantiser on the QKV weight (3072 x 9216, bf16) with a
    4096-token calibration batch: calibration maxima, smoothing, W_hat, the
    rank-32 range finder (4 power iterations) and residual packing (INT4 or
    MXFP4). Time per layer by HIP events around quantize_layer (its host work
    included)."""
    import statistics

    import numpy as np
    import torch

    import synth
    li = synth.make_layer(synth.CONFIGS["qkv"])
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    w, x = bf(li.w), bf(li.x)
    l = min(32 + 16, 3072)
    omega = torch.from_numpy(np.random.default_rng(0).standard_normal((9216, l))).to(dev)
    run = lambda: lib.quantize_layer(w, x, 32, omega=omega, fmt=fmt)
    run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        run()
        e.record()
        e.synchronize()
        ms.append(s.elapsed_time(e))
    return {"median_ms": round(statistics.median(ms), 3), "min_ms": round(min(ms), 3),
            "reps_ms": [round(v, 3) for v in ms]}


def mxfp4_block(lib, dev, iters=50):
    """The MXFP4 form on a transformer block's four linears at 4608 tokens
    (4096 image + 512 text): QKV 3072->9216, out 3072->3072, fc1 3072->12288
    with GELU, fc2 12288->3072 on fc1's output; rank 32. One step = activation
    quantisation + GEMM for each. Weights are random codes with E8M0
    exponents of a realistic range (kernel time does not depend on values)."""
    import statistics

    import torch

    from bit_quantized_diffusion_svdq_amd import pack_l1
    M, R = 4608, 32
    g = torch.Generator().manual_seed(21)

    def layer(K, N):
        G4 = (K // 64 + 3) // 4
        return dict(K=K, N=N,
                    inv=(torch.rand(K, generator=g) + 0.5).to(dev),
                    l1t=pack_l1((torch.randn((K, R), generator=g) * 0.05).to(torch.bfloat16)).to(dev),
                    l2t=(torch.randn((N, R), generator=g) * 0.1).to(torch.bfloat16).to(dev),
                    qw=torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8).to(dev),
                    sw=torch.randint(114, 122, (G4, N, 8), generator=g, dtype=torch.uint8).to(dev),
                    bias=(torch.randn(N, generator=g) * 0.02).to(torch.bfloat16).to(dev))
    L = [layer(3072, 9216), layer(3072, 3072), layer(3072, 12288), layer(12288, 3072)]
    xq = torch.randn((M, 3072), generator=g).to(torch.bfloat16).to(dev)
    xo = torch.randn((M, 3072), generator=g).to(torch.bfloat16).to(dev)
    xf = torch.randn((M, 3072), generator=g).to(torch.bfloat16).to(dev)
    ys = [torch.empty((M, l["N"]), dtype=torch.bfloat16, device=dev) for l in L]
    marks = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
             for _ in range(iters)]

    def run(li, x, act, y, mk):
        l = L[li]
        qx, sx, xl1 = lib.quantize_act_mxfp4(x, l["inv"], l["l1t"], R)
        if mk is not None:
            mk[0].record()
        lib.mxfp4_linear(qx, sx, xl1, l["qw"], l["sw"], l["l2t"], l["bias"], R, act=act, y=y)
        if mk is not None:
            mk[1].record()

    def step(i=None):
        mk = marks[i] if i is not None else [None] * 4
        run(0, xq, "none", ys[0], mk[0])
        run(1, xo, "none", ys[1], mk[1])
        run(2, xf, "gelu_tanh", ys[2], mk[2])
        run(3, ys[2], "none", ys[3], mk[3])

    for _ in range(20):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        step(i)
    e.record()
    e.synchronize()
    block_ms = s.elapsed_time(e) / iters
    gemm_ms = [sum(marks[i][k][0].elapsed_time(marks[i][k][1]) for i in range(iters)) / iters for k in range(4)]
    # the same block captured as one HIP graph (eight launches per step, five steps per graph)
    # and replayed: no host launch work between the kernels
    graph_ms = time_graph(step, 5, replays=10)
    ops = 2.0 * M * sum(l["K"] * l["N"] for l in L)
    gsum = sum(gemm_ms)
    # the same block with fc2's activation pass fused into fc1's epilogue
    # (svdq_gemm_mxfp4_quant_next: the bf16 hidden state is never stored)
    from bit_quantized_diffusion_svdq_amd import SvdqLinear, SvdqMLP
    lin = lambda l: SvdqLinear(l["inv"], l["l1t"], l["l2t"], l["qw"], l["sw"], l["bias"], R, fmt="mxfp4")
    mlp = SvdqMLP(lin(L[2]), lin(L[3]), M)
    mlp.x.copy_(xf)

    def step_fused():
        run(0, xq, "none", ys[0], None)
        run(1, xo, "none", ys[1], None)
        mlp._launches()

    for _ in range(10):
        step_fused()
    torch.cuda.synchronize()
    fused_ms, _ = time_reps(step_fused, 10, 5)
    fused_graph_ms = [time_graph(step_fused, 5, replays=10) for _ in range(3)]
    fmed, fgmed = statistics.median(fused_ms), statistics.median(fused_graph_ms)
    # the MXFP4 GEMM alone at the QKV shape of the headline (4096 tokens)
    Mq = 4096
    lq = L[0]
    xq4 = xq[:Mq].contiguous()
    qx4, sx4, xl4 = lib.quantize_act_mxfp4(xq4, lq["inv"], lq["l1t"], R)
    yq4 = torch.empty((Mq, lq["N"]), dtype=torch.bfloat16, device=dev)
    gq = lambda: lib.mxfp4_linear(qx4, sx4, xl4, lq["qw"], lq["sw"], lq["l2t"], lq["bias"], R, y=yq4)
    for _ in range(20):
        gq()
    qkv_ms, _ = time_reps(gq, 50, 5)
    qmed = statistics.median(qkv_ms)
    qkv_ops = 2.0 * Mq * lq["K"] * lq["N"]
    return {"M": M, "ops": ops, "block_us": round(block_ms * 1e3, 2),
            "block_fused_mlp_us": summary_us(fused_ms), "block_fused_mlp_graph_us": summary_us(fused_graph_ms),
            "block_fused_mlp_TOPS": round(ops / (fmed * 1e-3) / 1e12, 1),
            "block_fused_mlp_graph_TOPS": round(ops / (fgmed * 1e-3) / 1e12, 1),
            "qkv_gemm_M4096": {**summary_us(qkv_ms), "TOPS": round(qkv_ops / (qmed * 1e-3) / 1e12, 1),
                               "frac_of_fp4_peak": round(qkv_ops / (qmed * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4),
                               "frac_of_int8_peak": round(qkv_ops / (qmed * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)},
            "block_TOPS": round(ops / (block_ms * 1e-3) / 1e12, 1),
            "block_graph_us": round(graph_ms * 1e3, 2),
            "block_graph_TOPS": round(ops / (graph_ms * 1e-3) / 1e12, 1),
            "gemm_us": [round(x * 1e3, 2) for x in gemm_ms],
            "gemm_TOPS": round(ops / (gsum * 1e-3) / 1e12, 1),
            "gemm_frac_of_fp4_peak": round(ops / (gsum * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(M, K, N, rank, budget_s=20.0):
    """The oracle (numpy, fp64) timed on the host on a bounded sample of the
    QKV workload: the online path (activation quantisation + W4A4 output) for
    the first `rows` token rows, with every host thread BLAS offers and with
    one thread; scaled to effective TOPS."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import synth
    from oracle import svdq as osv
    cfg = synth.CONFIGS["qkv"]
    li = synth.make_layer(cfg)
    t0 = time.time()
    w = osv.prepare_svdq(li.x, li.w, li.bias, cfg.rank)
    t_prep = time.time() - t0

    def online(rows):
        qa = osv.quantize_act(li.x[:rows], w.inv_lambda, w.l1)
        osv.linear_output(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1, w.l2, w.bias)

    def measure(max_rows, share):
        rows = 16
        while True:
            t0 = time.perf_counter()
            online(rows)
            dt = time.perf_counter() - t0
            if dt >= share / 4 or rows >= max_rows:
                break
            rows *= 2
        reps = max(1, min(8, int(share / max(dt, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(reps):
            online(rows)
        dt = (time.perf_counter() - t0) / reps
        return rows, reps, dt

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    rows, reps, dt = measure(1024, budget_s * 0.6)
    with threadpool_limits(1):
        rows1, reps1, dt1 = measure(256, budget_s * 0.4)
    tops = lambda r, t: round(2.0 * r * cfg.N * cfg.K / t / 1e12, 6)
    return {"value": tops(rows, dt), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"online path (act quant + W4A4 output, fp64 numpy) on {rows} of {cfg.M} token rows "
                      f"of the QKV layer, mean of {reps} runs of {dt:.2f} s, {threads} threads; offline "
                      f"prepare (SVD etc.) {t_prep:.1f} s not included",
            "value_1thread": tops(rows1, dt1),
            "sample_1thread": f"{rows1} rows, mean of {reps1} runs of {dt1:.2f} s, 1 thread",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of back-to-back steps before the warm-up steps (clock settling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_diffusion_svdq_amd as lib
    lib.check_device(0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    clock = make_clock(lib, dev)

    M, K, N, R = 4096, 3072, 9216, 32
    log("preparing synthetic QKV operands")
    ops = synth_linear(M, K, N, R, seed=0, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    G4 = (K // 64 + 3) // 4
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((G4, M, 4), dtype=torch.float16, device=dev)
    xa = torch.empty((M, R), dtype=torch.float32, device=dev)

    def act():
        lib.svdq_quantize_act(ops["x"], M, K, K, ops["inv_lambda"], ops["l1t"], R, qa, sa, xa)

    def gemm():
        lib.svdq_gemm_w4a4(qa, sa, M, K, ops["qw"], ops["sw"], N, xa, ops["l2t"], R, ops["bias"], 0, y, 0, N)

    # the GEMM of every timed step is bracketed by HIP events on the stream it
    # is launched on (torch's current stream, which the binding passes down)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(max(args.steps, 1))]

    def step(i=None):
        act()
        if i is not None:
            marks[i][0].record()
        gemm()
        if i is not None:
            marks[i][1].record()

    # first run: the very first step of the process (code-object load, cold
    # caches, idle clock)
    f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    f0.record()
    act()
    f1.record()
    gemm()
    f2.record()
    f2.synchronize()
    first = {"step_us": round(f0.elapsed_time(f2) * 1e3, 1), "gemm_us": round(f1.elapsed_time(f2) * 1e3, 1)}
    mhz_idle = clock()
    n_settle = settle(step, args.settle_s)
    log(f"first step {first['step_us']} us; settled with {n_settle} steps ({args.settle_s} s)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # the timed steps carry no events: an event pair around each GEMM adds
    # 4-10 us of command-processor work per step that is no part of the layer
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mhz_timed = clock()
    ms = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms * 1e-3) / 1e12
    # the same K steps again, each GEMM bracketed by HIP events on its stream:
    # the GEMM's average launch duration inside the step (the roofline figure)
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    steps_ev_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    gemm_ms = sum(a.elapsed_time(b) for a, b in marks[:args.steps]) / args.steps
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    log(f"step {ms:.4f} ms, gemm {gemm_ms * 1e3:.1f} us ({gemm_tflops:.0f} TFLOP/s) at {mhz_timed} MHz")

    # GEMM alone: hot (operands resident in L2 / Infinity Cache) and rotated
    # over 4 operand sets (~400 MB: every launch reads HBM), 5 x 50 launches
    gemm_hot, mhz_hot = time_reps(gemm, 50, 5, clock)
    rot = []
    for k in range(4):
        o = synth_linear(M, K, N, R, seed=100 + k, device=dev)
        q2 = torch.empty_like(qa); s2 = torch.empty_like(sa); x2 = torch.empty_like(xa)
        lib.svdq_quantize_act(o["x"], M, K, K, o["inv_lambda"], o["l1t"], R, q2, s2, x2)
        rot.append((q2, s2, x2, o["qw"], o["sw"], o["l2t"], o["bias"], torch.empty_like(y)))
        del o
    ri = [0]

    def gemm_rot():
        q2, s2, x2, qw2, sw2, l22, b2, y2 = rot[ri[0] % 4]
        ri[0] += 1
        lib.svdq_gemm_w4a4(q2, s2, M, K, qw2, sw2, N, x2, l22, R, b2, 0, y2, 0, N)
    gemm_rot_ms, _ = time_reps(gemm_rot, 48, 5)
    del rot

    # activation kernel: hot (one X) and rotated over 12 copies of X (~300 MB)
    act_hot, _ = time_reps(act, 50, 5)
    xs = [ops["x"]] + [ops["x"].clone() for _ in range(11)]
    ai = [0]

    def act_rot():
        lib.svdq_quantize_act(xs[ai[0] % 12], M, K, K, ops["inv_lambda"], ops["l1t"], R, qa, sa, xa)
        ai[0] += 1
    act_rot_ms, _ = time_reps(act_rot, 48, 5)
    del xs

    # HBM reference: a plain device-to-device copy of known size (its counter
    # readings calibrate the GEMM's FETCH_SIZE / WRITE_SIZE figures)
    copy_bytes = 1 << 28
    csrc_buf = torch.ones(copy_bytes, dtype=torch.uint8, device=dev)
    cdst_buf = torch.empty_like(csrc_buf)
    copy_ms = time_events(lambda: cdst_buf.copy_(csrc_buf), 10)
    del csrc_buf, cdst_buf
    gemm_bytes = (M + N) * (K // 2 + (K // 64) * 2) + M * R * 4 + N * R * 2 + N * 2 + M * N * 2
    act_bytes = M * K * 2 + M * K // 2 + M * (K // 64) * 2 + M * R * 4 + K * 4 + R * K * 2
    import statistics
    act_med = statistics.median(act_rot_ms)
    props = torch.cuda.get_device_properties(dev)
    extra = {
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "hbm_GiB": round(props.total_memory / 2**30, 1), "hip": torch.version.hip,
                   "torch": torch.__version__, "library_version": lib.load_library().svdq_version()},
        "gemm_us": round(gemm_ms * 1e3, 2),
        "step_with_gemm_events_us": round(steps_ev_ms * 1e3, 2),
        "gemm_frac_of_int8_peak": round(gemm_tflops / PEAK_INT8_TOPS, 4),
        "sclk_MHz": {"idle_before": mhz_idle, "after_timed_steps": mhz_timed,
                     "after_gemm_reps": mhz_hot},
        "first_run": first,
        "settle": {"seconds": args.settle_s, "steps": n_settle},
        "gemm_hot": summary_us(gemm_hot),
        "gemm_rotated_4_sets": summary_us(gemm_rot_ms),
        "act_quant_hot": summary_us(act_hot),
        "act_quant_rotated_12_x": summary_us(act_rot_ms),
        "act_quant_GBps": round(act_bytes / (act_med * 1e-3) / 1e9, 1),
        "act_quant_hbm_frac": round(act_bytes / (act_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "copy_256MiB_GBps": round(2 * copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
    }

    if not args.no_extra:
        # AWQ W4A16 GEMV, weights rotated through 12 buffer sets (> 256 MB)
        Ma, Ka, Na = 4, 3072, 18432
        nrot = 12
        g = torch.Generator().manual_seed(5)
        xg = torch.randn((Ma, Ka), generator=g).to(torch.bfloat16).to(dev)
        inv_s = (1.0 / (torch.rand(Ka, generator=g) * 1.5 + 0.5)).to(dev)
        bufs = [dict(qw=torch.randint(0, 256, (Na, Ka // 2), generator=g, dtype=torch.uint8).to(dev),
                     sc=(torch.rand((Na, Ka // 64), generator=g) * 0.002 + 0.001).half().to(dev),
                     z=torch.randint(0, 16, (Na, Ka // 64), generator=g).half().to(dev))
                for _ in range(nrot)]
        ba = (torch.randn(Na, generator=g) * 0.02).to(torch.bfloat16).to(dev)
        ya = torch.empty((Ma, Na), dtype=torch.bfloat16, device=dev)
        it = [0]

        def gemv():
            b = bufs[it[0] % nrot]
            it[0] += 1
            lib.awq_gemv(xg, inv_s, b["qw"], b["sc"], b["z"], ba, y=ya)

        for _ in range(nrot * 2):
            gemv()
        gemv_graph = [time_graph(gemv, nrot * 8) for _ in range(5)]
        gemv_eager, _ = time_reps(gemv, 48, 5)
        # read-only floor: the same bytes (codes, scales, zero points) read once
        # per launch from the same rotated buffers, by the library's read probe
        sink = torch.empty(2048, dtype=torch.int32, device=dev)
        flat = [torch.cat([b["qw"].reshape(-1), b["sc"].view(torch.uint8).reshape(-1),
                           b["z"].view(torch.uint8).reshape(-1)]) for b in bufs]
        fi = [0]
        fbytes = flat[0].numel() // 16 * 16

        def readp():
            lib.svdq_probe_read(flat[fi[0] % nrot], fbytes, sink, 2048)
            fi[0] += 1
        floor_graph = [time_graph(readp, nrot * 8) for _ in range(5)]
        del flat
        gemv_bytes = Na * Ka // 2 + 2 * Na * (Ka // 64) * 2 + Ma * Ka * 2 + Ma * Na * 2 + Ka * 4 + Na * 2
        gmed = statistics.median(gemv_graph)
        fmed = statistics.median(floor_graph)
        extra.update({"awq_gemv_graph": summary_us(gemv_graph), "awq_gemv_eager": summary_us(gemv_eager),
                      "awq_gemv_us": round(gmed * 1e3, 2),
                      "awq_gemv_GBps": round(gemv_bytes / (gmed * 1e-3) / 1e9, 1),
                      "awq_gemv_hbm_frac": round(gemv_bytes / (gmed * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "read_only_floor_us": round(fmed * 1e3, 2),
                      "awq_gemv_frac_of_read_floor": round(fmed / gmed, 4)})
        del bufs
        # MLP pair: fc1 (GELU epilogue) -> fc2
        Mm = 4608
        fc1 = synth_linear(Mm, 3072, 12288, 32, seed=11, device=dev)
        fc2 = synth_linear(Mm, 12288, 3072, 32, seed=12, device=dev)
        h = torch.empty((Mm, 12288), dtype=torch.bfloat16, device=dev)
        y2 = torch.empty((Mm, 3072), dtype=torch.bfloat16, device=dev)

        def mlp():
            run_linear(lib, fc1, 32, act="gelu_tanh", y=h)
            fc2["x"] = h
            run_linear(lib, fc2, 32, y=y2)

        for _ in range(5):
            mlp()
        mlp_ms, _ = time_reps(mlp, 20, 5)
        mlp_flops = 2.0 * Mm * 3072 * 12288 * 2
        mm = statistics.median(mlp_ms)
        extra.update({"mlp_pair": summary_us(mlp_ms),
                      "mlp_pair_TOPS": round(mlp_flops / (mm * 1e-3) / 1e12, 1)})
        log(f"gemv {gmed * 1e3:.2f} us (read floor {fmed * 1e3:.2f}), mlp pair {mm * 1e3:.1f} us")
        # the same MLP with fc2's activation pass fused into fc1's epilogue
        # (the bf16 hidden state never stored), eager and as one graph; and
        # the unfused pair as a graph
        from bit_quantized_diffusion_svdq_amd import SvdqLinear, SvdqMLP
        lin = lambda o: SvdqLinear(o["inv_lambda"], o["l1t"], o["l2t"], o["qw"], o["sw"], o["bias"], 32)
        blk = SvdqMLP(lin(fc1), lin(fc2), Mm)
        blk.x.copy_(fc1["x"])
        fused = lambda: blk.forward(blk.x)
        for _ in range(5):
            fused()
        fused_ms, _ = time_reps(fused, 20, 5)
        fused_graph = [time_graph(blk._launches, 10) for _ in range(5)]
        pair_graph = [time_graph(mlp, 10) for _ in range(5)]
        fm = statistics.median(fused_ms)
        extra.update({"mlp_fused": summary_us(fused_ms), "mlp_fused_graph": summary_us(fused_graph),
                      "mlp_pair_graph": summary_us(pair_graph),
                      "mlp_fused_TOPS": round(mlp_flops / (fm * 1e-3) / 1e12, 1)})
        log(f"mlp fused {fm * 1e3:.1f} us (graph {statistics.median(fused_graph) * 1e3:.1f}, "
            f"unfused graph {statistics.median(pair_graph) * 1e3:.1f})")
        del fc1, fc2, h, y2, blk
        extra["offline_quantize_qkv"] = offline_quantize_timing(lib, dev)
        extra["offline_quantize_qkv_mxfp4"] = offline_quantize_timing(lib, dev, fmt="mxfp4")
        log(f"offline quantiser, QKV layer: {extra['offline_quantize_qkv']['median_ms']} ms")
        extra["mxfp4_block"] = mxfp4_block(lib, dev)
        log(f"mxfp4 block {extra['mxfp4_block']['block_us']} us, with the fused MLP "
            f"{extra['mxfp4_block']['block_fused_mlp_us']['median_us']} us")

    out = {
        "metric": "W4A4 linear effective TOPS (M4096 K3072 N9216 r32) + % of MI355X MFMA peak",
        "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4 x int4 (exact on fp6 MFMA), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "DiT attention QKV projection as an SVDQuant W4A4 linear: act quant + "
                               "INT4 g64 GEMM + rank-32 low-rank + bias, bf16 out",
                   "M": M, "K": K, "N": N, "rank": R, "group": 64, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP6_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP6_TFLOPS, 4),
                     "traffic": gemm_traffic_bytes(), "traffic_unit": "HBM bytes per launch",
                     "algorithmic_bytes": gemm_bytes, "kernel": "gemm_w4a4_kernel"},
        "frac_of_int8_peak_step": round(value / PEAK_INT8_TOPS, 4),
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(M, K, N, R)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
