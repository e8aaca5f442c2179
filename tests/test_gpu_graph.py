"""A transformer block's MXFP4 linears (QKV 3072 -> 9216, out 3072 -> 3072,
fc1 3072 -> 12288 with GELU, fc2 12288 -> 3072 on fc1's output; 4608 tokens,
rank 32) captured into one HIP graph with the library's CapturedSequence.

Every replay must give outputs bit-identical to the eager launches (the graph
holds the same launches); replays are interleaved with eager work and
synchronisations and each one is checked. The eager outputs themselves meet
the oracle on sampled rows, element by element: within half a bf16 ulp of
the fp64 result plus 1e-4 of its rms (the fp32 accumulation and GELU), GELU
included."""
import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4 as omx
from gpu_util import assert_bf16_output, dev_u16, host_bf16_f64, host_u16, note, sample_rows

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib


def _layer(K, N, seed, x_bits=None):
    cfg = synth.LayerConfig("blk", M=4608, K=K, N=N, rank=32, n_outliers=31, outlier_factor=30.0, seed=seed)
    li = synth.make_layer(cfg)
    x = li.x if x_bits is None else x_bits
    return x, omx.prepare_mx(x, li.w, li.bias, 32)


def test_mx_block_graph_replay_matches_eager():
    from test_gpu_mxfp4 import DevMx
    note("mxfp4 block graph capture")
    M, R = 4608, 32
    specs = [(3072, 9216, 101), (3072, 3072, 102), (3072, 12288, 103)]
    layers = [_layer(K, N, s) for (K, N, s) in specs]
    dws = [DevMx(w) for _, w in layers]
    xs = [dev_u16(x) for x, _ in layers]
    # fc2 is calibrated on a stand-in of fc1's output distribution (its own
    # input at run time is fc1's output buffer)
    x2_cal = synth.make_matrix_bf16(M, 12288, seed=104, std=0.4)
    li2 = synth.make_layer(synth.LayerConfig("fc2", M=8, K=12288, N=3072, rank=R, seed=105))
    w2 = omx.prepare_mx(x2_cal, li2.w, li2.bias, R)
    d2 = DevMx(w2)
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for (_, N, _) in specs]
    y2 = torch.empty((M, 3072), dtype=torch.bfloat16, device="cuda")
    G4 = lambda K: (K // 64 + 3) // 4
    bufs = [(torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((G4(K), M, 8), dtype=torch.uint8, device="cuda"),
             torch.empty((M, R), dtype=torch.float32, device="cuda")) for K in (3072, 3072, 3072, 12288)]
    acts = ["none", "none", "gelu_tanh"]

    def block():
        for i in range(3):
            qx, sx, xl1 = bufs[i]
            lib.svdq_quantize_act_mxfp4(xs[i], M, 3072, 3072, dws[i].inv_lambda, dws[i].l1t, R, qx, sx, xl1)
            lib.mxfp4_linear(qx, sx, xl1, dws[i].qw, dws[i].sw, dws[i].l2t, dws[i].bias, R, act=acts[i], y=ys[i])
        qx, sx, xl1 = bufs[3]
        lib.svdq_quantize_act_mxfp4(ys[2], M, 12288, 12288, d2.inv_lambda, d2.l1t, R, qx, sx, xl1)
        lib.mxfp4_linear(qx, sx, xl1, d2.qw, d2.sw, d2.l2t, d2.bias, R, y=y2)

    block()
    torch.cuda.synchronize()
    eager = [t.clone() for t in ys + [y2]]
    g = lib.CapturedSequence(block)
    for rep in range(3):
        for t in ys + [y2]:
            t.fill_(0)                       # a replay must rewrite every output
        junk = torch.randn((1024, 1024), device="cuda") @ torch.randn((1024, 1024), device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ys + [y2], eager)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}, output {i}"
        del junk
    # the eager outputs against the oracle on sampled rows
    rows = sample_rows(M, 2, 10, 9)
    for i, (x, w) in enumerate(layers):
        qa = omx.quantize_act(x[rows], w.inv_lambda, w.l1)
        y64 = omx.linear_output(qa.codes, qa.exps, w.qw_codes, w.qw_exps, qa.xl1, w.l2, w.bias, acts[i])
        note(f"mxfp4 block graph: layer {i} against the oracle")
        assert_bf16_output(host_bf16_f64(eager[i])[rows], y64, 1e-4)
    h = host_u16(eager[2])
    qa = omx.quantize_act(h[rows], w2.inv_lambda, w2.l1)
    y64 = omx.linear_output(qa.codes, qa.exps, w2.qw_codes, w2.qw_exps, qa.xl1, w2.l2, w2.bias)
    assert_bf16_output(host_bf16_f64(eager[3])[rows], y64, 1e-4)
