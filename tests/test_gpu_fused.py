"""fc2's activation pass fused into fc1's GEMM epilogue (INT4 and MXFP4),
and the MLP block recorded into a HIP graph.

Bars: the fused codes and scales are bit-identical to the activation
kernel's on fc1's bf16 output H (and to the oracle's activation pass on
that H); xl1 of the fused pass agrees with the oracle's fp64 definition on
that H to 1e-4 relative (its fp32 partial sums run in a different order
than the activation kernel's); stores stay inside their arrays (sentinel
guard bands); the graph replays the eager block bit for bit, and the block's
output meets the bf16 output bar of the oracle's fc2 on the GPU's H."""
import numpy as np
import pytest
import torch

import synth
from oracle import svdq as osv
from gpu_util import DevSvdq, dev, dev_u16, host_u16, note, rel_fro, assert_bf16_output

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib

SENT = 0x5A


def _fc1(M, K, N, r, seed):
    x = synth.make_matrix_bf16(M, K, seed=seed, std=1.0)
    w = synth.make_matrix_bf16(K, N, seed=seed + 1, std=0.05)
    b = synth.make_matrix_bf16(1, N, seed=seed + 2, std=0.02)[0]
    return x, DevSvdq(osv.prepare_svdq(x, w, b, r))


def _next_layer(K2, r2, seed):
    """the next layer's activation-side arrays: inv_lambda and L1 (random)"""
    rng = np.random.default_rng(seed)
    inv = rng.uniform(0.3, 2.0, K2).astype(np.float32)
    l1 = synth.bf16_round((rng.standard_normal((K2, r2)) * 0.05).astype(np.float32)) if r2 else None
    return inv, l1


def _sentinel(n):
    return torch.full((n,), SENT, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("M,K,N,r,r2", [(200, 512, 1024, 16, 32), (64, 256, 384, 0, 16), (130, 320, 256, 32, 0),
                                        (128, 192, 512, 32, 64), (257, 3072, 12288, 32, 32), (1, 128, 128, 16, 16),
                                        (33, 64, 640, 0, 48)],
                         ids=lambda v: str(v))
def test_fused_activation_pass_matches_unfused(M, K, N, r, r2):
    note(f"fused next act M={M} K={K} N={N} r={r} r2={r2}")
    x, d1 = _fc1(M, K, N, r, seed=M + N)
    inv2, l1_2 = _next_layer(N, r2, seed=N + r2)
    inv2_d = dev(inv2)
    l1t2 = dev_u16(osv.pack_l1_tiles(l1_2)) if r2 else None
    qx, sx, xl1 = lib.quantize_act(dev_u16(x), d1.inv_lambda, d1.l1t, r)
    # unfused: H, then the activation kernel on it
    h = lib.w4a4_linear(qx, sx, xl1, d1.qw, d1.sw, d1.l2t, d1.bias, r, act="gelu_tanh")
    qa, sa, la = lib.quantize_act(h, inv2_d, l1t2, r2)
    # fused, into views of sentinel-filled buffers
    G4 = (N // 64 + 3) // 4
    nq, ns, nl = M * N // 2, G4 * M * 8, M * r2 * 4
    bq, bs, bl = _sentinel(nq + 4096), _sentinel(ns + 4096), _sentinel(nl + 4096)
    out = (bq[:nq].view(M, N // 2), bs[:ns].view(torch.float16).view(G4, M, 4),
           bl[:nl].view(torch.float32).view(M, r2) if r2 else None)
    qf, sf, lf = lib.w4a4_linear_quant_next(qx, sx, xl1, d1.qw, d1.sw, d1.l2t, d1.bias, r, "gelu_tanh", inv2_d,
                                            l1t2, r2, out=out)
    torch.cuda.synchronize()
    for name, b, n in (("qx", bq, nq), ("sx", bs, ns), ("xl1", bl, nl)):
        tail = b[n:].cpu().numpy()
        assert np.all(tail == SENT), f"{np.count_nonzero(tail != SENT)} bytes written past {name}"
    assert torch.equal(qf, qa)
    if (N // 64) % 4 == 0:
        assert torch.equal(sf.view(torch.int16), sa.view(torch.int16))
    else:                      # padding groups of the last quad are not written by the fused pass
        G = N // 64
        assert torch.equal(sf.view(torch.int16)[:-1], sa.view(torch.int16)[:-1])
        assert torch.equal(sf.view(torch.int16)[-1, :, :G % 4], sa.view(torch.int16)[-1, :, :G % 4])
    # the oracle's activation pass on the GPU's H
    ref = osv.quantize_act(host_u16(h), inv2, l1_2)
    assert np.array_equal(qf.cpu().numpy(), ref.qx)
    assert np.array_equal(osv.unpack_scales(sf.cpu().numpy(), N // 64).view(np.uint16), ref.sx.view(np.uint16))
    if r2:
        lfn = lf.cpu().numpy()
        assert rel_fro(lfn, ref.xl1) <= 1e-4
        assert rel_fro(lfn, la.cpu().numpy()) <= 1e-5


def _mlp(M, K1, N1, N2, r1, r2, seed):
    x = synth.make_matrix_bf16(M, K1, seed=seed, std=1.0)
    w1 = synth.make_matrix_bf16(K1, N1, seed=seed + 1, std=0.05)
    b1 = synth.make_matrix_bf16(1, N1, seed=seed + 2, std=0.02)[0]
    o1 = osv.prepare_svdq(x, w1, b1, r1)
    # fc2 calibrated on the oracle's H of fc1 (a chained MLP)
    _, y1 = osv.forward(o1, x, act="gelu_tanh")
    h_ref = osv.output_bf16(y1)
    w2 = synth.make_matrix_bf16(N1, N2, seed=seed + 3, std=0.05)
    b2 = synth.make_matrix_bf16(1, N2, seed=seed + 4, std=0.02)[0]
    o2 = osv.prepare_svdq(h_ref, w2, b2, r2)
    return x, o1, o2


def _linear(o):
    d = DevSvdq(o)
    return lib.SvdqLinear(d.inv_lambda, d.l1t, d.l2t, d.qw, d.sw, d.bias, o.rank)


def test_mlp_block_graph_replay_and_oracle():
    M, K1, N1, N2 = 256, 512, 1024, 512
    note(f"mlp block M={M} {K1}->{N1}->{N2}")
    x, o1, o2 = _mlp(M, K1, N1, N2, 16, 32, seed=41)
    mlp = lib.SvdqMLP(_linear(o1), _linear(o2), M)
    xd = dev_u16(x)
    y_eager = mlp.forward(xd).clone()
    mlp.capture()
    for rep in range(3):
        mlp.y.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        y_g = mlp.replay(xd)
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep} differs"
    # the unfused chain (H stored, then the activation kernel)
    f1, f2 = mlp.fc1, mlp.fc2
    qx, sx, xl1 = lib.quantize_act(xd, f1.inv_lambda, f1.l1t, f1.rank)
    h = lib.w4a4_linear(qx, sx, xl1, f1.qw, f1.sw, f1.l2t, f1.bias, f1.rank, act="gelu_tanh")
    q2, s2, l2 = lib.quantize_act(h, f2.inv_lambda, f2.l1t, f2.rank)
    y_u = lib.w4a4_linear(q2, s2, l2, f2.qw, f2.sw, f2.l2t, f2.bias, f2.rank)
    assert torch.equal(q2, mlp.qx2) and torch.equal(s2.view(torch.int16), mlp.sx2.view(torch.int16))
    assert rel_fro(y_eager.float().cpu().numpy(), y_u.float().cpu().numpy()) <= 1e-3
    # the oracle's fc2 on the GPU's H, sampled rows
    rows = np.array([0, 1, 77, 128, 200, 255])
    hb = host_u16(h)[rows]
    _, y64 = osv.forward(o2, hb)
    assert_bf16_output(y_eager.float().cpu().numpy()[rows], y64, 1e-4)


def test_mlp_full_size_fused_codes_and_sampled_rows():
    """fc1 3072 -> 12288 with GELU, fc2's pass fused, at 4608 tokens: the
    fused codes and scales equal the activation kernel's on the stored H; xl1
    equals the oracle's on sampled rows."""
    M, K, N, r, r2 = 4608, 3072, 12288, 32, 32
    note(f"fused next act full size M={M} K={K} N={N}")
    x, d1 = _fc1(M, K, N, r, seed=7)
    inv2, l1_2 = _next_layer(N, r2, seed=8)
    inv2_d, l1t2 = dev(inv2), dev_u16(osv.pack_l1_tiles(l1_2))
    qx, sx, xl1 = lib.quantize_act(dev_u16(x), d1.inv_lambda, d1.l1t, r)
    h = lib.w4a4_linear(qx, sx, xl1, d1.qw, d1.sw, d1.l2t, d1.bias, r, act="gelu_tanh")
    qa, sa, la = lib.quantize_act(h, inv2_d, l1t2, r2)
    qf, sf, lf = lib.w4a4_linear_quant_next(qx, sx, xl1, d1.qw, d1.sw, d1.l2t, d1.bias, r, "gelu_tanh", inv2_d,
                                            l1t2, r2)
    torch.cuda.synchronize()
    assert torch.equal(qf, qa) and torch.equal(sf.view(torch.int16), sa.view(torch.int16))
    rows = np.array([0, 127, 128, 2047, 4607])
    ref = osv.quantize_act(host_u16(h)[rows], inv2, l1_2)
    assert rel_fro(lf.cpu().numpy()[rows], ref.xl1) <= 1e-4
    assert rel_fro(lf.cpu().numpy(), la.cpu().numpy()) <= 1e-5


# ---------------------------------------------------------------- MXFP4 form

def _fc1_mx(M, K, N, r, seed):
    from oracle import mxfp4 as omx
    from test_gpu_mxfp4 import DevMx
    x = synth.make_matrix_bf16(M, K, seed=seed, std=1.0)
    w = synth.make_matrix_bf16(K, N, seed=seed + 1, std=0.05)
    b = synth.make_matrix_bf16(1, N, seed=seed + 2, std=0.02)[0]
    return x, DevMx(omx.prepare_mx(x, w, b, r))


def _check_mx_scales(sf, sa, N):
    """E8M0 records equal except the padding blocks of a last partial quad,
    which the fused pass does not write"""
    G = N // 64
    if G % 4 == 0:
        assert torch.equal(sf, sa)
    else:
        assert torch.equal(sf[:-1], sa[:-1])
        for gq in range(G % 4):
            assert torch.equal(sf[-1, :, gq], sa[-1, :, gq]) and torch.equal(sf[-1, :, 4 + gq], sa[-1, :, 4 + gq])


@pytest.mark.parametrize("M,K,N,r,r2", [(200, 512, 1024, 16, 32), (64, 256, 384, 0, 16), (130, 320, 256, 32, 0),
                                        (128, 192, 512, 32, 64), (257, 3072, 12288, 32, 32), (1, 128, 128, 16, 16),
                                        (33, 64, 640, 0, 48)],
                         ids=lambda v: str(v))
def test_fused_mxfp4_activation_pass_matches_unfused(M, K, N, r, r2):
    from oracle import mxfp4 as omx
    note(f"fused next act mxfp4 M={M} K={K} N={N} r={r} r2={r2}")
    x, d1 = _fc1_mx(M, K, N, r, seed=M + N + 1)
    inv2, l1_2 = _next_layer(N, r2, seed=N + r2 + 1)
    inv2_d = dev(inv2)
    l1t2 = dev_u16(osv.pack_l1_tiles(l1_2)) if r2 else None
    qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(x), d1.inv_lambda, d1.l1t, r)
    h = lib.mxfp4_linear(qx, sx, xl1, d1.qw, d1.sw, d1.l2t, d1.bias, r, act="gelu_tanh")
    qa, sa, la = lib.quantize_act_mxfp4(h, inv2_d, l1t2, r2)
    G4 = (N // 64 + 3) // 4
    nq, ns, nl = M * N // 2, G4 * M * 8, M * r2 * 4
    bq, bs, bl = _sentinel(nq + 4096), _sentinel(ns + 4096), _sentinel(nl + 4096)
    out = (bq[:nq].view(M, N // 2), bs[:ns].view(G4, M, 8),
           bl[:nl].view(torch.float32).view(M, r2) if r2 else None)
    qf, sf, lf = lib.mxfp4_linear_quant_next(qx, sx, xl1, d1.qw, d1.sw, d1.l2t, d1.bias, r, "gelu_tanh", inv2_d,
                                             l1t2, r2, out=out)
    torch.cuda.synchronize()
    for name, b, n in (("qx", bq, nq), ("sx", bs, ns), ("xl1", bl, nl)):
        tail = b[n:].cpu().numpy()
        assert np.all(tail == SENT), f"{np.count_nonzero(tail != SENT)} bytes written past {name}"
    assert torch.equal(qf, qa)
    _check_mx_scales(sf, sa, N)
    # the oracle's MXFP4 activation pass on the GPU's H
    ref = omx.quantize_act(host_u16(h), inv2, l1_2)
    assert np.array_equal(qf.cpu().numpy(), omx.pack_fp4(ref.codes))
    assert np.array_equal(omx.unpack_scales(sf.cpu().numpy(), N // 32), ref.exps)
    if r2:
        lfn = lf.cpu().numpy()
        assert rel_fro(lfn, ref.xl1) <= 1e-4
        assert rel_fro(lfn, la.cpu().numpy()) <= 1e-5


def test_mlp_block_mxfp4_graph_replay_and_oracle():
    from oracle import mxfp4 as omx
    from test_gpu_mxfp4 import DevMx
    M, K1, N1, N2, r1, r2 = 256, 512, 1024, 512, 16, 32
    note(f"mlp block mxfp4 M={M} {K1}->{N1}->{N2}")
    x = synth.make_matrix_bf16(M, K1, seed=43, std=1.0)
    w1 = synth.make_matrix_bf16(K1, N1, seed=44, std=0.05)
    b1 = synth.make_matrix_bf16(1, N1, seed=45, std=0.02)[0]
    o1 = omx.prepare_mx(x, w1, b1, r1)
    _, y1 = omx.forward(o1, x, act="gelu_tanh")
    w2 = synth.make_matrix_bf16(N1, N2, seed=46, std=0.05)
    b2 = synth.make_matrix_bf16(1, N2, seed=47, std=0.02)[0]
    o2 = omx.prepare_mx(osv.output_bf16(y1), w2, b2, r2)

    def linear(o):
        d = DevMx(o)
        return lib.SvdqLinear(d.inv_lambda, d.l1t, d.l2t, d.qw, d.sw, d.bias, o.rank, fmt="mxfp4")

    mlp = lib.SvdqMLP(linear(o1), linear(o2), M)
    xd = dev_u16(x)
    y_eager = mlp.forward(xd).clone()
    mlp.capture()
    for rep in range(3):
        mlp.y.zero_()
        torch.cuda.synchronize()
        y_g = mlp.replay(xd)
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep} differs"
    f1, f2 = mlp.fc1, mlp.fc2
    qx, sx, xl1 = lib.quantize_act_mxfp4(xd, f1.inv_lambda, f1.l1t, f1.rank)
    h = lib.mxfp4_linear(qx, sx, xl1, f1.qw, f1.sw, f1.l2t, f1.bias, f1.rank, act="gelu_tanh")
    q2, s2, l2 = lib.quantize_act_mxfp4(h, f2.inv_lambda, f2.l1t, f2.rank)
    y_u = lib.mxfp4_linear(q2, s2, l2, f2.qw, f2.sw, f2.l2t, f2.bias, f2.rank)
    assert torch.equal(q2, mlp.qx2) and torch.equal(s2, mlp.sx2)
    assert rel_fro(y_eager.float().cpu().numpy(), y_u.float().cpu().numpy()) <= 1e-3
    rows = np.array([0, 1, 77, 128, 200, 255])
    _, y64 = omx.forward(o2, host_u16(h)[rows])
    assert_bf16_output(y_eager.float().cpu().numpy()[rows], y64, 1e-4)
