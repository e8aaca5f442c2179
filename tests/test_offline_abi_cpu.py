"""Host-side checks of the offline quantiser's C ABI (no GPU needed): every
malformed call returns its documented status before touching the device;
well-formed calls on a machine without a gfx950 GPU stop at the capability
check. The workspace query is pure host arithmetic."""
import ctypes

import pytest

import bit_quantized_diffusion_svdq_amd as svdq

OK, NULL, SHAPE, ALIGN, UNSUP, DEVICE = 0, 1, 2, 3, 4, 5
A, B, C, D, E = 0x7F0000000000, 0x7F0000100000, 0x7F0000200000, 0x7F0000300000, 0x7F0000400000


@pytest.fixture(scope="module")
def lib():
    return svdq.load_library()


def _no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")


@pytest.mark.parametrize("kw,status", [
    (dict(axis=2), UNSUP), (dict(acc=3), UNSUP), (dict(cols=100), SHAPE), (dict(lda=8), SHAPE),
    (dict(lda=260), SHAPE), (dict(rows=-1), SHAPE), (dict(out=None), NULL), (dict(a=None), NULL),
    (dict(a=A + 8), ALIGN), (dict(out=B + 2), ALIGN),
])
def test_calib_absmax_rejects(lib, kw, status):
    a = dict(a=A, rows=64, cols=256, lda=256, axis=0, acc=0, out=B)
    a.update(kw)
    assert lib.svdq_calib_absmax(a["a"], a["rows"], a["cols"], a["lda"], a["axis"], a["acc"], a["out"], None) == status


def test_calib_absmax_empty_is_ok(lib):
    assert lib.svdq_calib_absmax(None, 0, 0, 0, 0, 0, None, None) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(alpha=-0.1), UNSUP), (dict(alpha=1.5), UNSUP), (dict(alpha=float("nan")), UNSUP), (dict(K=-1), SHAPE),
    (dict(ax=None), NULL), (dict(inv=None), NULL), (dict(aw=B + 2), ALIGN),
])
def test_smoothing_rejects(lib, kw, status):
    a = dict(ax=A, aw=B, K=256, alpha=0.5, inv=C)
    a.update(kw)
    assert lib.svdq_smoothing(a["ax"], a["aw"], a["K"], a["alpha"], a["inv"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(N=100), SHAPE), (dict(ldw=8), SHAPE), (dict(K=70000), SHAPE), (dict(w=None), NULL),
    (dict(w_hat=None), NULL), (dict(w=A + 8), ALIGN), (dict(w_hat=C + 8), ALIGN),
])
def test_smooth_weight_rejects(lib, kw, status):
    a = dict(w=A, K=256, N=512, ldw=512, inv=B, w_hat=C)
    a.update(kw)
    assert lib.svdq_smooth_weight(a["w"], a["K"], a["N"], a["ldw"], a["inv"], a["w_hat"], None) == status


def _ws(lib, K, N, r, l):
    out = ctypes.c_int64(0)
    st = lib.svdq_lowrank_workspace_size(K, N, r, l, ctypes.byref(out))
    return st, out.value


def test_lowrank_workspace_size(lib):
    st, n = _ws(lib, 3072, 9216, 32, 48)
    assert st == OK and n >= 8 * (2 * 3072 * 48 + 2 * 9216 * 48)
    st2, n2 = _ws(lib, 512, 512, 16, 32)
    assert st2 == OK and 0 < n2 < n
    assert lib.svdq_lowrank_workspace_size(512, 512, 16, 32, None) == NULL


@pytest.mark.parametrize("K,N,r,l", [(512, 512, 0, 16), (512, 512, 24, 32), (512, 512, 96, 96),
                                     (512, 512, 32, 16), (512, 512, 32, 89), (64, 512, 32, 80),
                                     (512, 40, 32, 48), (0, 512, 16, 16)])
def test_lowrank_shape_rejects(lib, K, N, r, l):
    assert _ws(lib, K, N, r, l)[0] == SHAPE


@pytest.mark.parametrize("kw,status", [
    (dict(iters=-1), SHAPE), (dict(iters=65), SHAPE), (dict(wsb=1024), SHAPE), (dict(w_hat=None), NULL),
    (dict(omega=None), NULL), (dict(l1=None), NULL), (dict(ws=None), NULL), (dict(ws=E + 8), ALIGN),
    (dict(omega=B + 4), ALIGN),
])
def test_lowrank_rejects(lib, kw, status):
    a = dict(w_hat=A, K=512, N=512, r=16, omega=B, l=32, iters=4, l1=C, l2=D, sigma=None, ws=E, wsb=1 << 30)
    a.update(kw)
    assert lib.svdq_lowrank(a["w_hat"], a["K"], a["N"], a["r"], a["omega"], a["l"], a["iters"], a["l1"], a["l2"],
                            a["sigma"], a["ws"], a["wsb"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), SHAPE), (dict(N=0), SHAPE), (dict(r=128), SHAPE), (dict(r=8), SHAPE), (dict(qw=None), NULL),
    (dict(l1=None), NULL), (dict(sw=None), NULL), (dict(qw=C + 4), ALIGN), (dict(w_hat=A + 4), ALIGN),
])
def test_quantize_residual_rejects(lib, kw, status):
    a = dict(w_hat=A, K=256, N=64, l1=B, l2=E, r=16, qw=C, sw=D)
    a.update(kw)
    assert lib.svdq_quantize_residual(a["w_hat"], a["K"], a["N"], a["l1"], a["l2"], a["r"], a["qw"], a["sw"],
                                      None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), SHAPE), (dict(N=0), SHAPE), (dict(r=128), SHAPE), (dict(r=8), SHAPE), (dict(qw=None), NULL),
    (dict(l1=None), NULL), (dict(sw=None), NULL), (dict(qw=C + 8), ALIGN), (dict(w_hat=A + 4), ALIGN),
])
def test_quantize_residual_mxfp4_rejects(lib, kw, status):
    a = dict(w_hat=A, K=256, N=64, l1=B, l2=E, r=16, qw=C, sw=D)
    a.update(kw)
    assert lib.svdq_quantize_residual_mxfp4(a["w_hat"], a["K"], a["N"], a["l1"], a["l2"], a["r"], a["qw"], a["sw"],
                                            None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(K=192), SHAPE), (dict(K=0), SHAPE), (dict(N=24), SHAPE), (dict(N=0), SHAPE), (dict(ldw=48), SHAPE),
    (dict(w=None), NULL), (dict(qwt=None), NULL), (dict(scale=None), NULL), (dict(zero=None), NULL),
    (dict(qwt=C + 8), ALIGN), (dict(w=A + 1), ALIGN), (dict(inv_s=B + 2), ALIGN), (dict(zero=E + 1), ALIGN),
])
def test_awq_quantize_weight_rejects(lib, kw, status):
    a = dict(w=A, K=256, N=64, ldw=64, inv_s=B, qwt=C, scale=D, zero=E)
    a.update(kw)
    assert lib.awq_quantize_weight(a["w"], a["K"], a["N"], a["ldw"], a["inv_s"], a["qwt"], a["scale"], a["zero"],
                                   None) == status


def test_awq_quantize_weight_without_gpu_reports_device_error(lib):
    _no_gpu()
    assert lib.awq_quantize_weight(A, 256, 64, 64, None, C, D, E, None) == DEVICE


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), SHAPE), (dict(r=20), SHAPE), (dict(N=0), SHAPE), (dict(l1t=None), NULL), (dict(l1t=C + 2), ALIGN),
])
def test_pack_lowrank_rejects(lib, kw, status):
    a = dict(l1=A, l2=B, K=256, N=64, r=16, l1t=C, l2t=D)
    a.update(kw)
    assert lib.svdq_pack_lowrank(a["l1"], a["l2"], a["K"], a["N"], a["r"], a["l1t"], a["l2t"], None) == status


def test_rank_zero_residual_and_pack_need_no_factors(lib):
    _no_gpu()
    assert lib.svdq_pack_lowrank(None, None, 256, 64, 0, None, None, None) == OK
    assert lib.svdq_quantize_residual(A, 256, 64, None, None, 0, C, D, None) == DEVICE
    assert lib.svdq_quantize_residual_mxfp4(A, 256, 64, None, None, 0, C, D, None) == DEVICE


def test_valid_offline_calls_without_gpu_report_device_error(lib):
    _no_gpu()
    assert lib.svdq_calib_absmax(A, 64, 256, 256, 1, 0, B, None) == DEVICE
    assert lib.svdq_smoothing(A, B, 256, 0.5, C, None) == DEVICE
    assert lib.svdq_smooth_weight(A, 256, 512, 512, B, C, None) == DEVICE
    assert lib.svdq_lowrank(A, 512, 512, 16, B, 32, 4, C, D, None, E, 1 << 30, None) == DEVICE
    assert lib.svdq_pack_lowrank(A, B, 256, 64, 16, C, D, None) == DEVICE


def test_quantize_layer_rejects_host_tensors():
    import torch
    w = torch.zeros((256, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        svdq.quantize_layer(w, w.T.contiguous(), 16)            # calibration batch of the wrong width
    with pytest.raises(ValueError, match="rank"):
        svdq.quantize_layer(w, None, 24, smooth=False)
    with pytest.raises(ValueError, match="GPU"):
        svdq.quantize_layer(w, torch.zeros((8, 256), dtype=torch.bfloat16), 16)


# ---------------------------------------------------------------- fused next-layer pass

def _next(lib, entry="svdq_gemm_w4a4_quant_next", **kw):
    a = dict(qx=A, sx=B, M=128, K=256, qw=C, sw=D, N=256, xl1=E, l2t=E + 0x10000, rank=16, bias=None, act=1,
             inv=A + 0x20000, l1t=B + 0x20000, r2=32, qxn=C + 0x20000, sxn=D + 0x20000, xl1n=E + 0x20000,
             ws=A + 0x80000, wsb=1 << 30)
    a.update(kw)
    return getattr(lib, entry)(a["qx"], a["sx"], a["M"], a["K"], a["qw"], a["sw"], a["N"], a["xl1"],
                               a["l2t"], a["rank"], a["bias"], a["act"], a["inv"], a["l1t"], a["r2"],
                               a["qxn"], a["sxn"], a["xl1n"], a["ws"], a["wsb"], None)


NEXT_ENTRIES = ["svdq_gemm_w4a4_quant_next", "svdq_gemm_mxfp4_quant_next"]


@pytest.mark.parametrize("entry", NEXT_ENTRIES)
@pytest.mark.parametrize("kw,status", [
    (dict(N=200), SHAPE), (dict(N=192), SHAPE), (dict(K=96), SHAPE), (dict(r2=80), SHAPE), (dict(r2=8), SHAPE),
    (dict(rank=20), SHAPE), (dict(act=5), UNSUP), (dict(wsb=100), SHAPE), (dict(inv=None), NULL),
    (dict(l1t=None), NULL), (dict(ws=None), NULL), (dict(qxn=None), NULL), (dict(xl1=None), NULL),
    (dict(inv=A + 4), ALIGN), (dict(l1t=B + 2), ALIGN), (dict(qxn=C + 8), ALIGN), (dict(M=-1), SHAPE),
])
def test_quant_next_rejects(lib, entry, kw, status):
    assert _next(lib, entry, **kw) == status


def test_quant_next_scale_alignment_by_format(lib):
    """INT4 scales are fp16 (2-byte aligned); MXFP4 exponents are bytes."""
    assert _next(lib, "svdq_gemm_w4a4_quant_next", sxn=D + 0x20001) == ALIGN
    assert _next(lib, "svdq_gemm_mxfp4_quant_next", sxn=D + 0x20001) in (OK, DEVICE)


def test_quant_next_workspace_and_empty(lib):
    out = ctypes.c_int64(0)
    assert lib.svdq_gemm_w4a4_quant_next_workspace_size(4608, 12288, 32, ctypes.byref(out)) == OK
    assert out.value == 96 * 4608 * 32 * 4
    assert lib.svdq_gemm_w4a4_quant_next_workspace_size(4608, 12288, 0, ctypes.byref(out)) == OK and out.value == 0
    assert lib.svdq_gemm_w4a4_quant_next_workspace_size(64, 100, 16, ctypes.byref(out)) == SHAPE
    assert _next(lib, M=0) == OK
    assert _next(lib, r2=0, l1t=None, xl1n=None, ws=None, wsb=0) in (OK, DEVICE)


@pytest.mark.parametrize("entry", NEXT_ENTRIES)
def test_quant_next_without_gpu_reports_device_error(lib, entry):
    _no_gpu()
    assert _next(lib, entry) == DEVICE


def test_noalloc_refuses_beyond_scratch_on_the_host(lib):
    """The allocation-free fused GEMM checks its partials against the built-in
    64 MiB before touching any device."""
    st = lib.svdq_gemm_w4a4_quant_next_noalloc(A, B, 8192, 256, C, D, 12288, E, E + 0x10000, 16, None, 1,
                                               A + 0x20000, B + 0x20000, 64, C + 0x20000, D + 0x20000, E + 0x20000,
                                               None)
    assert st == SHAPE and b"scratch" in lib.svdq_last_error()
    assert lib.svdq_gemm_w4a4_quant_next_noalloc(A, B, 128, 256, C, D, 200, E, E, 16, None, 1, A, B, 32,
                                                 C, D, E, None) == SHAPE
