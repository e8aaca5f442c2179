"""The allocation-free fused GEMM (svdq_gemm_w4a4_quant_next_noalloc)
against the workspace form, through the C ABI: two calls in a row on the
same built-in scratch, the second smaller, each bit-identical to the
workspace form on the same inputs; and a size past the scratch is refused."""
import numpy as np
import pytest
import torch

from gpu_util import note

pytestmark = pytest.mark.gpu

import bit_quantized_diffusion_svdq_amd as lib
from bit_quantized_diffusion_svdq_amd import _lib


def _operands(M, K, N, r, r2, seed):
    g = torch.Generator().manual_seed(seed)
    d = "cuda"
    G4, G4n = (K // 64 + 3) // 4, (N // 64 + 3) // 4
    op = dict(
        qx=torch.randint(0, 256, (M, K // 2), generator=g, dtype=torch.uint8).to(d),
        sx=(torch.rand((G4, M, 4), generator=g) * 0.02 + 0.005).half().to(d),
        qw=torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8).to(d),
        sw=(torch.rand((G4, N, 4), generator=g) * 0.02 + 0.005).half().to(d),
        xl1=(torch.randn((M, r), generator=g)).to(d) if r else None,
        l2t=(torch.randn((N, r), generator=g) * 0.05).to(torch.bfloat16).to(d) if r else None,
        bias=(torch.randn(N, generator=g) * 0.02).to(torch.bfloat16).to(d),
        inv=(torch.rand(N, generator=g) * 1.5 + 0.3).to(d),
        l1t=(torch.randn(N * r2, generator=g) * 0.05).to(torch.bfloat16).to(d) if r2 else None,
    )
    outs = lambda: (torch.empty((M, N // 2), dtype=torch.uint8, device=d),
                    torch.empty((G4n, M, 4), dtype=torch.float16, device=d),
                    torch.empty((M, r2), dtype=torch.float32, device=d) if r2 else None)
    return op, outs


def _both(M, K, N, r, r2, seed):
    note(f"no-alloc fused gemm M={M} K={K} N={N} r={r} r2={r2}")
    op, outs = _operands(M, K, N, r, r2, seed)
    a, b = outs(), outs()
    nb = lib.svdq_gemm_w4a4_quant_next_workspace_size(M, N, r2)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    args = (op["qx"], op["sx"], M, K, op["qw"], op["sw"], N, op["xl1"], op["l2t"], r, op["bias"], 1,
            op["inv"], op["l1t"], r2)
    lib.svdq_gemm_w4a4_quant_next(*args, *a, ws, nb)
    _lib.svdq_gemm_w4a4_quant_next_noalloc(*args, *b)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    if r2:
        assert torch.equal(a[2].view(torch.int32), b[2].view(torch.int32))


def test_noalloc_matches_workspace_form_two_calls():
    _both(4608, 3072, 12288, 32, 32, seed=1)      # the MLP's fc1: 56.6 MB of partials
    _both(200, 512, 1024, 16, 32, seed=2)         # then a smaller call on the same scratch


def test_noalloc_refuses_partials_beyond_its_scratch():
    note("no-alloc refusal (host check, nothing launched)")
    L = lib.load_library()
    st = L.svdq_gemm_w4a4_quant_next_noalloc(0x1000, 0x1000, 8192, 256, 0x1000, 0x1000, 12288, 0x1000, 0x1000, 16,
                                             None, 1, 0x1000, 0x1000, 64, 0x1000, 0x1000, 0x1000, None)
    assert st == 2 and b"scratch" in L.svdq_last_error()
