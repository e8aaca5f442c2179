"""Guard bands: every kernel writes its outputs and nothing else.

Each output is a view into a larger allocation filled with a sentinel byte
pattern: rows past M (128 of them, a whole tile), columns past N up to the
leading dimension, and bytes past the end of the dense arrays. After the
call every byte outside the view must still hold the sentinel, and the
values inside must equal those of a call on tightly allocated outputs.
Ragged M and N (not multiples of the 128 x 128 tile), group counts that are
not a multiple of 4, ranks 0 / 16 / 48, INT4 and MXFP4, bf16 and fp32."""
import numpy as np
import pytest
import torch

import synth
from oracle import svdq as osv
from gpu_util import DevSvdq, dev_u16, note

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib

SENT = 0x5A          # sentinel byte
SHAPES = [(77, 192, 200, 0), (130, 320, 136, 16), (300, 704, 264, 48), (1, 64, 16, 16)]


def sentinel(nbytes):
    return torch.full((nbytes,), SENT, dtype=torch.uint8, device="cuda")


def untouched(buf, lo, hi=None):
    """bytes [lo, hi) of a uint8 buffer still hold the sentinel"""
    b = buf[lo:hi].cpu().numpy()
    return bool(np.all(b == SENT)), int(np.count_nonzero(b != SENT))


def layer(M, K, N, r):
    x = synth.make_matrix_bf16(M, K, seed=M + 1, std=1.0)
    wb = synth.make_matrix_bf16(K, N, seed=N + 2, std=0.05)
    b = synth.make_matrix_bf16(1, N, seed=5, std=0.02)[0]
    return x, wb, b


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_K%d_N%d_r%d" % s)
def test_gemm_stores_stay_inside(fmt, out, shape):
    M, K, N, r = shape
    note(f"guard gemm {fmt} {out} M={M} K={K} N={N} r={r}")
    x, wb, b = layer(M, K, N, r)
    if fmt == "int4":
        dw = DevSvdq(osv.prepare_svdq(x, wb, b, r))
        qx, sx, xl1 = lib.quantize_act(dev_u16(x), dw.inv_lambda, dw.l1t, r)
        gemm = lib.w4a4_linear
    else:
        from oracle import mxfp4 as omx
        from test_gpu_mxfp4 import DevMx
        dw = DevMx(omx.prepare_mx(x, wb, b, r))
        qx, sx, xl1 = lib.quantize_act_mxfp4(dev_u16(x), dw.inv_lambda, dw.l1t, r)
        gemm = lib.mxfp4_linear
    esz = 2 if out == torch.bfloat16 else 4
    ldy = N + 24                                   # a multiple of 8 beyond N
    rows = M + 128
    buf = sentinel(rows * ldy * esz + 256)
    yv = buf[:rows * ldy * esz].view(out).view(rows, ldy)[:M, :N]
    assert yv.stride(0) == ldy
    gemm(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, r, y=yv)
    yt = gemm(qx, sx, xl1, dw.qw, dw.sw, dw.l2t, dw.bias, r, out_dtype=out)
    torch.cuda.synchronize()
    ok, n = untouched(buf, M * ldy * esz)          # rows >= M and the tail
    assert ok, f"{n} bytes written past row M"
    b2 = buf[:M * ldy * esz].view(M, ldy * esz)[:, N * esz:].cpu().numpy()
    assert np.all(b2 == SENT), f"{np.count_nonzero(b2 != SENT)} bytes written past column N"
    assert torch.equal(yv.contiguous().view(torch.uint8), yt.view(torch.uint8))


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_K%d_N%d_r%d" % s)
def test_act_stores_stay_inside(fmt, shape):
    M, K, _, r = shape
    note(f"guard act {fmt} M={M} K={K} r={r}")
    x = synth.make_matrix_bf16(M, K, seed=M + 9, std=2.0)
    rng = np.random.default_rng(M)
    inv = torch.from_numpy(rng.uniform(0.3, 2.0, K).astype(np.float32)).cuda()
    l1 = (torch.randn((K, r), generator=torch.Generator().manual_seed(3)) * 0.1).to(torch.bfloat16)
    l1t = lib.pack_l1(l1).cuda() if r else None
    G4 = (K // 64 + 3) // 4
    sxe = 8                                         # bytes per (quad, row): 4 fp16 or 8 E8M0
    nq, ns, nl = M * K // 2, G4 * M * sxe, M * r * 4
    bq, bs, bl = sentinel(nq + 4096), sentinel(ns + 4096), sentinel(nl + 4096)
    qx = bq[:nq].view(M, K // 2)
    if fmt == "int4":
        sx = bs[:ns].view(torch.float16).view(G4, M, 4)
        fn, raw = lib.quantize_act, lib.svdq_quantize_act
    else:
        sx = bs[:ns].view(G4, M, 8)
        fn, raw = lib.quantize_act_mxfp4, lib.svdq_quantize_act_mxfp4
    xl1 = bl[:nl].view(torch.float32).view(M, r) if r else None
    xd = dev_u16(x)
    raw(xd, M, K, K, inv, l1t, r, qx, sx, xl1)
    qt, st, lt = fn(xd, inv, l1t, r)
    torch.cuda.synchronize()
    for name, b, n in (("qx", bq, nq), ("sx", bs, ns), ("xl1", bl, nl)):
        ok, cnt = untouched(b, n)
        assert ok, f"{cnt} bytes written past the end of {name}"
    assert torch.equal(qx, qt) and torch.equal(sx.view(torch.uint8), st.view(torch.uint8))
    if r:
        assert torch.equal(xl1.view(torch.int32), lt.view(torch.int32))


@pytest.mark.parametrize("M,K,N", [(1, 256, 48), (4, 3072, 18432), (7, 640, 1040), (16, 128, 16)])
def test_gemv_stores_stay_inside(M, K, N):
    from oracle import awq as oawq
    note(f"guard awq M={M} K={K} N={N}")
    cfg = synth.LayerConfig("g", M=M, K=K, N=N, kind="awq", seed=M + N)
    li = synth.make_layer(cfg)
    aw = oawq.prepare_awq(li.w, li.chan_scale, li.bias)
    ny = M * N * 2
    buf = sentinel(ny + 65536)
    yv = buf[:ny].view(torch.bfloat16).view(M, N)
    args = (dev_u16(li.x), torch.from_numpy(aw.inv_s).cuda(), torch.from_numpy(aw.qwt).cuda(),
            torch.from_numpy(aw.scale_t).cuda(), torch.from_numpy(aw.zero_t).cuda(), dev_u16(aw.bias))
    lib.awq_gemv(*args, N=N, y=yv)
    yt = lib.awq_gemv(*args, N=N)
    torch.cuda.synchronize()
    ok, cnt = untouched(buf, ny)
    assert ok, f"{cnt} bytes written past the end of y"
    assert torch.equal(yv.view(torch.int16), yt.view(torch.int16))
