"""Benchmark: SVDQuant W4A4 linear on one MI355X.

Step = one forward of the DiT attention QKV projection as a W4A4 linear:
svdq_quantize_act (smoothing + rank-32 down-projection + INT4 g64 activation
quantisation) followed by svdq_gemm_w4a4 (group GEMM + low-rank up-projection
+ bias, bf16 out), M=4096 tokens, K=3072, N=9216, rank 32. `value` is the
effective TOPS of that linear, 2*M*N*K / step time.

In the same run (separate timed loops, reported under "extra"): the AWQ W4A16
adaLN GEMV (4 x 3072 -> 18432, weights rotated through more buffers than the
256 MB Infinity Cache holds, so every launch reads HBM) and the MLP pair
(fc1 3072 -> 12288 with the GELU epilogue, then fc2 12288 -> 3072, 4608 tokens).

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
# the plain device copy this script also runs.  The figures hold only for the
# kernel sources they were taken on (their sha256 below); otherwise the
# traffic is reported as null.
GEMM_TRAFFIC = {
    "source_sha256": "bf40777b0a807bfba2ab9ffcda60dbd0d1b831a18449a5a694cf92fdf741250e",
    "fetch_kib": 66638.78, "write_kib": 74732.45,        # QKV GEMM, mean of 40 dispatches
    "fetch_factor": 262144.0 / 131084.49,                 # 256 MiB copy: known bytes / FETCH_SIZE
    "write_factor": 262144.0 / 262144.0,                  # 256 MiB copy: known bytes / WRITE_SIZE
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


def mxfp4_block(lib, dev, iters=50):
    """The MXFP4 form on a transformer block's four linears at 4608 tokens
    (4096 image + 512 text): QKV 3072->9216, out 3072->3072, fc1 3072->12288
    with GELU, fc2 12288->3072 on fc1's output; rank 32. One step = activation
    quantisation + GEMM for each. Weights are random codes with E8M0
    exponents of a realistic range (kernel time does not depend on values)."""
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
    return {"M": M, "ops": ops, "block_us": round(block_ms * 1e3, 2),
            "block_TOPS": round(ops / (block_ms * 1e-3) / 1e12, 1),
            "block_graph_us": round(graph_ms * 1e3, 2),
            "block_graph_TOPS": round(ops / (graph_ms * 1e-3) / 1e12, 1),
            "gemm_us": [round(x * 1e3, 2) for x in gemm_ms],
            "gemm_TOPS": round(ops / (gsum * 1e-3) / 1e12, 1),
            "gemm_frac_of_fp4_peak": round(ops / (gsum * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4)}


def cpu_baseline(M, K, N, rank, budget_s=20.0):
    """The oracle (numpy, fp64) timed on the host on a bounded sample of the
    QKV workload: the online path (activation quantisation + W4A4 output) for
    the first `rows` token rows; scaled to effective TOPS."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import svdq as osv
    cfg = synth.CONFIGS["qkv"]
    li = synth.make_layer(cfg)
    t0 = time.time()
    w = osv.prepare_svdq(li.x, li.w, li.bias, cfg.rank)
    t_prep = time.time() - t0
    rows = 32
    while True:
        t0 = time.perf_counter()
        qa = osv.quantize_act(li.x[:rows], w.inv_lambda, w.l1)
        osv.linear_output(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1, w.l2, w.bias)
        dt = time.perf_counter() - t0
        if dt >= 2.0 or rows >= 1024:
            break
        rows *= 2
    reps = max(1, int(budget_s / max(dt, 1e-3) / 2))
    reps = min(reps, 8)
    t0 = time.perf_counter()
    for _ in range(reps):
        qa = osv.quantize_act(li.x[:rows], w.inv_lambda, w.l1)
        osv.linear_output(qa.codes, qa.sx, w.qw_codes, w.sw, qa.xl1, w.l2, w.bias)
    dt = (time.perf_counter() - t0) / reps
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(2.0 * rows * cfg.N * cfg.K / dt / 1e12, 6), "unit": "TOPS",
            "cores": threads, "kind": "oracle",
            "sample": f"online path (act quant + W4A4 output, fp64 numpy) on {rows} of {cfg.M} token rows "
                      f"of the QKV layer, mean of {reps} runs of {dt:.2f} s; offline prepare "
                      f"(SVD etc.) {t_prep:.1f} s not included"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=1000)
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

    M, K, N, R = 4096, 3072, 9216, 32
    log("preparing synthetic QKV operands")
    ops = synth_linear(M, K, N, R, seed=0, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qx, sx, xl1 = lib.quantize_act(ops["x"], ops["inv_lambda"], ops["l1t"], R)

    # the GEMM of every timed step is bracketed by HIP events on the stream it
    # is launched on (torch's current stream, which the binding passes down)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]

    def step(i=None):
        qa, sa, xa = lib.quantize_act(ops["x"], ops["inv_lambda"], ops["l1t"], R)
        if i is not None:
            marks[i][0].record()
        lib.w4a4_linear(qa, sa, xa, ops["qw"], ops["sw"], ops["l2t"], ops["bias"], R, y=y)
        if i is not None:
            marks[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms * 1e-3) / 1e12
    gemm_ms = sum(a.elapsed_time(b) for a, b in marks) / args.steps

    qx_b = torch.empty_like(qx)
    sx_b = torch.empty_like(sx)
    xl1_b = torch.empty_like(xl1)
    act_ms = time_graph(lambda: lib.svdq_quantize_act(ops["x"], M, K, K, ops["inv_lambda"], ops["l1t"], R,
                                                      qx_b, sx_b, xl1_b), 50)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    # HBM reference: a plain device-to-device copy of known size (its counter
    # readings calibrate the GEMM's FETCH_SIZE / WRITE_SIZE figures)
    copy_bytes = 1 << 28
    csrc_buf = torch.ones(copy_bytes, dtype=torch.uint8, device=dev)
    cdst_buf = torch.empty_like(csrc_buf)
    copy_ms = time_events(lambda: cdst_buf.copy_(csrc_buf), 10)
    del csrc_buf, cdst_buf
    gemm_bytes = (M + N) * (K // 2 + (K // 64) * 2) + M * R * 4 + N * R * 2 + N * 2 + M * N * 2
    act_bytes = M * K * 2 + M * K // 2 + M * (K // 64) * 2 + M * R * 4 + K * 4 + R * K * 2
    log(f"step {ms:.4f} ms, gemm {gemm_ms * 1e3:.1f} us ({gemm_tflops:.0f} TFLOP/s), "
        f"act {act_ms * 1e3:.1f} us")

    extra = {"gemm_us": round(gemm_ms * 1e3, 2), "act_quant_us": round(act_ms * 1e3, 2),
             "act_quant_GBps": round(act_bytes / (act_ms * 1e-3) / 1e9, 1),
             "act_quant_hbm_frac": round(act_bytes / (act_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "gemm_frac_of_int8_peak": round(gemm_tflops / PEAK_INT8_TOPS, 4),
             "copy_256MiB_GBps": round(2 * copy_bytes / (copy_ms * 1e-3) / 1e9, 1)}

    if not args.no_extra:
        # AWQ W4A16 GEMV, weights rotated through > 256 MB
        Ma, Ka, Na = 4, 3072, 18432
        nrot = 12
        g = torch.Generator().manual_seed(5)
        xa = torch.randn((Ma, Ka), generator=g).to(torch.bfloat16).to(dev)
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
            lib.awq_gemv(xa, inv_s, b["qw"], b["sc"], b["z"], ba, y=ya)

        for _ in range(nrot * 2):
            gemv()
        gemv_ms = time_graph(gemv, nrot * 8)
        gemv_bytes = Na * Ka // 2 + 2 * Na * (Ka // 64) * 2 + Ma * Ka * 2 + Ma * Na * 2 + Ka * 4 + Na * 2
        extra.update({"awq_gemv_us": round(gemv_ms * 1e3, 2),
                      "awq_gemv_GBps": round(gemv_bytes / (gemv_ms * 1e-3) / 1e9, 1),
                      "awq_gemv_hbm_frac": round(gemv_bytes / (gemv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
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
        mlp_ms = time_events(mlp, 50)
        mlp_flops = 2.0 * Mm * 3072 * 12288 * 2
        extra.update({"mlp_pair_us": round(mlp_ms * 1e3, 2),
                      "mlp_pair_TOPS": round(mlp_flops / (mlp_ms * 1e-3) / 1e12, 1)})
        log(f"gemv {gemv_ms * 1e3:.2f} us, mlp pair {mlp_ms * 1e3:.1f} us")
        del fc1, fc2, h, y2
        extra["mxfp4_block"] = mxfp4_block(lib, dev)
        log(f"mxfp4 block {extra['mxfp4_block']['block_us']} us")

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
