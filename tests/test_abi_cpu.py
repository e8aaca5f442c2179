"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/svdq.h declares, and rejects malformed arguments
with the documented status before touching the device (the remio.ai page,
hardware section: unsupported combinations must raise clear errors rather
than run incompatible kernels)."""
import ctypes
import os
import re

import pytest

import bit_quantized_diffusion_svdq_amd as svdq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, UNSUP, DEVICE = 0, 1, 2, 3, 4, 5

# fake but well-aligned device addresses: validation must reject bad calls
# before any of them is dereferenced or passed to HIP
A = 0x7F0000000000
B = 0x7F0000100000
C = 0x7F0000200000
D = 0x7F0000300000
E = 0x7F0000400000


@pytest.fixture(scope="module")
def lib():
    return svdq.load_library()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "svdq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"svdq_quantize_act", "svdq_gemm_w4a4", "awq_gemv_w4a16", "svdq_gemm_w4a4_partials",
            "svdq_quantize_act_mxfp4", "svdq_gemm_mxfp4",
            "svdq_check_device", "svdq_status_string", "svdq_last_error", "svdq_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(7):
        assert lib.svdq_status_string(s)
    assert lib.svdq_status_string(99) == b"unknown status"
    assert lib.svdq_version() == 404


def _act(lib, **kw):
    a = dict(x=A, M=128, K=256, ldx=256, inv=None, l1t=B, rank=16, qx=C, sx=D, xl1=E)
    a.update(kw)
    return lib.svdq_quantize_act(a["x"], a["M"], a["K"], a["ldx"], a["inv"], a["l1t"], a["rank"],
                                 a["qx"], a["sx"], a["xl1"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), SHAPE), (dict(K=0), SHAPE), (dict(M=-1), SHAPE), (dict(rank=8), SHAPE),
    (dict(rank=144), SHAPE), (dict(ldx=128), SHAPE), (dict(ldx=260), ALIGN),
    (dict(x=None), NULL), (dict(qx=None), NULL), (dict(sx=None), NULL),
    (dict(l1t=None), NULL), (dict(xl1=None), NULL), (dict(x=A + 2), ALIGN), (dict(qx=C + 8), ALIGN),
    (dict(K=1 << 20), SHAPE),
])
def test_quantize_act_rejects(lib, kw, status):
    assert _act(lib, **kw) == status
    assert lib.svdq_last_error()


def test_quantize_act_stride_and_lds_limits(lib):
    """Row strides from 2^26 elements are refused; ranks up to 32 take any K
    (the LDS-staged form's LDS does not grow with K), the register form for
    larger ranks is bounded by its LDS."""
    big = 1 << 26
    assert _act(lib, ldx=big) == SHAPE and b"2^26" in lib.svdq_last_error()
    assert _act(lib, K=21888, ldx=21888, rank=128) == SHAPE
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: well-formed calls on these placeholder pointers would launch")
    assert _act(lib, K=40000, ldx=40000, rank=32) == DEVICE
    assert _act(lib, K=21824, ldx=21824, rank=128) == DEVICE


def _gemm(lib, **kw):
    a = dict(qx=A, sx=B, M=64, K=256, qw=C, sw=D, N=128, xl1=E, l2t=E + 4096, rank=16,
             bias=None, act=0, y=E + 65536, ydt=0, ldy=128)
    a.update(kw)
    return lib.svdq_gemm_w4a4(a["qx"], a["sx"], a["M"], a["K"], a["qw"], a["sw"], a["N"], a["xl1"],
                              a["l2t"], a["rank"], a["bias"], a["act"], a["y"], a["ydt"], a["ldy"],
                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=100), SHAPE), (dict(N=0), SHAPE), (dict(K=96), SHAPE), (dict(ldy=64), SHAPE),
    (dict(ldy=132), ALIGN), (dict(act=2), UNSUP), (dict(ydt=3), UNSUP), (dict(qw=None), NULL),
    (dict(y=None), NULL), (dict(xl1=None), NULL), (dict(rank=20), SHAPE), (dict(qw=C + 4), ALIGN),
    (dict(y=E + 65536 + 8), ALIGN), (dict(M=1 << 20, K=4096), SHAPE), (dict(N=1 << 20, K=4096), SHAPE),
    (dict(M=1 << 22, K=64, rank=128), SHAPE), (dict(N=1 << 23, K=64, rank=128), SHAPE),
    (dict(sx=B + 8), ALIGN), (dict(sw=D + 8), ALIGN), (dict(M=1 << 23, K=64, N=256, ldy=256), SHAPE),
])
def test_gemm_rejects(lib, kw, status):
    assert _gemm(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(m0=-1), SHAPE), (dict(mcount=100), SHAPE), (dict(n0=64, ncount=100), SHAPE),
    (dict(p=None), NULL), (dict(K=65), SHAPE), (dict(M=1 << 20, K=4096), SHAPE),
])
def test_partials_rejects(lib, kw, status):
    a = dict(qx=A, M=64, K=256, qw=C, N=128, m0=0, mcount=64, n0=0, ncount=128, p=E)
    a.update(kw)
    assert lib.svdq_gemm_w4a4_partials(a["qx"], a["M"], a["K"], a["qw"], a["N"], a["m0"],
                                       a["mcount"], a["n0"], a["ncount"], a["p"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), SHAPE), (dict(M=17), SHAPE), (dict(N=40), SHAPE), (dict(K=48), SHAPE),
    (dict(K=192), SHAPE),                      # group pairs: K must be a multiple of 128
    (dict(zero=None), NULL), (dict(x=A + 4), ALIGN), (dict(scale=C + 1), ALIGN),
    (dict(N=1 << 20, K=4096), SHAPE),          # packed weights of 2 GiB: beyond 31-bit offsets
])
def test_gemv_rejects(lib, kw, status):
    a = dict(x=A, M=4, K=256, inv=None, qw=B, scale=C, zero=D, N=64, bias=None, y=E)
    a.update(kw)
    assert lib.awq_gemv_w4a16(a["x"], a["M"], a["K"], a["inv"], a["qw"], a["scale"], a["zero"],
                              a["N"], a["bias"], a["y"], None) == status


def test_valid_arguments_without_gpu_report_device_error(lib):
    """Well-formed calls on a machine without a gfx950 GPU stop at the
    capability check (never a silent fallback)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _act(lib) == DEVICE
    assert b"device" in lib.svdq_last_error().lower()
    assert _gemm(lib) == DEVICE
    assert lib.svdq_check_device(0) == DEVICE
    with pytest.raises(svdq.SvdqError):
        svdq.check_device(0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import bit_quantized_diffusion_svdq_amd._lib as L
    monkeypatch.setattr(L, "_LIB", None)
    monkeypatch.setattr(L, "library_path", lambda: str(tmp_path / "libsvdq.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        L.load_library()


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), SHAPE), (dict(N=100), SHAPE), (dict(qw=None), NULL), (dict(sx=B + 8), ALIGN),
    (dict(act=2), UNSUP), (dict(M=1 << 20, K=4096), SHAPE),
])
def test_mxfp4_entry_points_validate_like_int4(lib, kw, status):
    a = dict(qx=A, sx=B, M=64, K=256, qw=C, sw=D, N=128, xl1=E, l2t=E + 4096, rank=16,
             bias=None, act=0, y=E + 65536, ydt=0, ldy=128)
    a.update(kw)
    assert lib.svdq_gemm_mxfp4(a["qx"], a["sx"], a["M"], a["K"], a["qw"], a["sw"], a["N"], a["xl1"],
                               a["l2t"], a["rank"], a["bias"], a["act"], a["y"], a["ydt"], a["ldy"],
                               None) == status
    q = dict(x=A, M=128, K=256, ldx=256, inv=None, l1t=B, rank=16, qx=C, sx=D, xl1=E)
    if "K" in kw and kw["K"] == 96:
        q["K"], q["ldx"] = 96, 96
        assert lib.svdq_quantize_act_mxfp4(q["x"], q["M"], q["K"], q["ldx"], q["inv"], q["l1t"], q["rank"],
                                           q["qx"], q["sx"], q["xl1"], None) == SHAPE


# ---------------------------------------------------------------- layer descriptions

def _desc(**kw):
    a = dict(K=3072, N=9216, rank=32, group=64, fmt="int4", act="none")
    a.update(kw)
    return svdq.layer_desc(**a)


@pytest.mark.parametrize("kw", [{}, dict(fmt="mxfp4"), dict(rank=0), dict(rank=128), dict(act="gelu_tanh"),
                                dict(K=64, N=8), dict(K=12288, N=3072)])
def test_validate_desc_accepts(kw):
    assert svdq.svdq_validate_desc(_desc(**kw)) == OK


@pytest.mark.parametrize("kw,status,word", [
    (dict(K=3000), SHAPE, "K"), (dict(K=0), SHAPE, "K"), (dict(K=-64), SHAPE, "K"),
    (dict(N=9220), SHAPE, "N"), (dict(N=0), SHAPE, "N"),
    (dict(rank=8), SHAPE, "rank"), (dict(rank=144), SHAPE, "rank"), (dict(rank=-16), SHAPE, "rank"),
    (dict(group=128), UNSUP, "group"), (dict(group=32), UNSUP, "group"),
    (dict(fmt=2), UNSUP, "format"), (dict(fmt=-1), UNSUP, "format"),
    (dict(act=7), UNSUP, "activation"),
])
def test_validate_desc_rejects(lib, kw, status, word):
    assert svdq.svdq_validate_desc(_desc(**kw)) == status
    assert word in lib.svdq_last_error().decode()
    with pytest.raises(svdq.SvdqError):
        svdq.validate_desc(_desc(**kw))


def test_validate_desc_null(lib):
    assert svdq.svdq_validate_desc(None) == NULL
    assert lib.svdq_layer_sizes_of(None, None) == NULL


def test_layer_sizes():
    s = svdq.layer_sizes(_desc())
    assert s == dict(qw=9216 * 1536, sw=12 * 9216 * 8, l1t=3072 * 32 * 2, l2t=9216 * 32 * 2,
                     inv_lambda=3072 * 4, bias=9216 * 2, qx_row=1536, sx_row=96, xl1_row=128)
    # K = 192: three groups round up to one quad of scales
    s = svdq.layer_sizes(_desc(K=192, N=16, rank=0, fmt="mxfp4"))
    assert (s["sw"], s["sx_row"], s["l1t"], s["l2t"]) == (16 * 8, 8, 0, 0)
    with pytest.raises(svdq.SvdqError):
        svdq.layer_sizes(_desc(group=16))


# ---------------------------------------------------------------- binding argument checks
# (raised in Python before any C call, so they run without a GPU)

def test_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):          # host tensors never reach a kernel
        svdq.quantize_act(x, None, None, 0)
    with pytest.raises(ValueError, match="bfloat16"):
        svdq.quantize_act(x.float(), None, None, 0)
    with pytest.raises(ValueError, match="contiguous columns"):
        svdq.quantize_act(torch.zeros((4, 512), dtype=torch.bfloat16)[:, ::2], None, None, 0)
    with pytest.raises(ValueError, match="l1t"):
        svdq.quantize_act(x, None, torch.zeros(10, dtype=torch.bfloat16), 16)
    qx = torch.zeros((4, 128), dtype=torch.uint8)
    sx = torch.zeros((1, 4, 4), dtype=torch.float16)
    qw = torch.zeros((8, 128), dtype=torch.uint8)
    sw = torch.zeros((1, 8, 4), dtype=torch.float16)
    with pytest.raises(ValueError, match="qw"):            # K of the weights differs
        svdq.w4a4_linear(qx, sx, None, torch.zeros((8, 64), dtype=torch.uint8), sw, None, None, 0)
    with pytest.raises(ValueError, match="y must be bf16 or fp32"):
        svdq.w4a4_linear(qx, sx, None, qw, sw, None, None, 0, y=torch.zeros((4, 8), dtype=torch.float16))
    with pytest.raises(ValueError, match="sw"):
        svdq.w4a4_linear(qx, sx, None, qw, sw[:, :4], None, None, 0)
    with pytest.raises(ValueError, match="bias"):
        svdq.w4a4_linear(qx, sx, None, qw, sw, None, torch.zeros(7, dtype=torch.bfloat16), 0)
    with pytest.raises(ValueError, match="sx"):            # INT4 scales given to the MXFP4 GEMM
        svdq.mxfp4_linear(qx, sx, None, qw, sw, None, None, 0)
    with pytest.raises(ValueError, match="qwt"):
        svdq.awq_gemv(x, None, torch.zeros(10, dtype=torch.uint8), torch.zeros(64, dtype=torch.float16),
                      torch.zeros(64, dtype=torch.float16), None, N=16)
