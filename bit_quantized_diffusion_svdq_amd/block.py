"""Layers and an MLP block over the library's entry points, with every
buffer allocated up front so that a forward can be recorded into a HIP graph
and replayed.

The MLP (fc1 with GELU, then fc2) is the transformer part the pages name
with attention as where the time goes (remio.ai page, section on SVDQuant
moving hard values out of 4-bit: attention and feed-forward projections
dominate). Its forward is three launches: fc1's activation pass, fc1's GEMM
whose epilogue runs fc2's activation pass on the bf16 GELU output (the
16-bit hidden state never goes to memory), and fc2's GEMM. Removing launch
and graph overhead is the gain the donmalab.com page reports for compiled
pipelines (section on squeezing out more performance); the block records its
launches into one graph (CapturedSequence).

Marshalling only: the arithmetic is the library's.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib
from .graph import CapturedSequence


@dataclass
class SvdqLinear:
    """One SVDQ W4A4 layer's device arrays in the library's layouts."""
    inv_lambda: torch.Tensor        # fp32 [K]
    l1t: torch.Tensor | None        # bf16, L1 tile layout (K * rank values)
    l2t: torch.Tensor | None        # bf16 [N, rank]
    qw: torch.Tensor                # uint8 [N, K/2]
    sw: torch.Tensor                # fp16 [ceil(K/256), N, 4] (INT4) or uint8 [ceil(K/256), N, 8] (MXFP4)
    bias: torch.Tensor | None       # bf16 [N]
    rank: int
    fmt: str = "int4"               # "int4" (group 64, fp16 scales) or "mxfp4" (E2M1, E8M0 per 32)

    @property
    def K(self) -> int:
        return self.qw.shape[1] * 2

    @property
    def N(self) -> int:
        return self.qw.shape[0]

    @classmethod
    def from_quantized(cls, d: dict) -> "SvdqLinear":
        """From the dict quantize_layer() returns."""
        r = d["rank"]
        return cls(d["inv_lambda"], d["l1t"] if r else None, d["l2t"] if r else None, d["qw"], d["sw"],
                   d.get("bias"), r, d.get("fmt", "int4"))

    def __call__(self, x: torch.Tensor, act: str = "none", out_dtype=torch.bfloat16, y=None,
                 stream=None) -> torch.Tensor:
        """Y for bf16 activations x [M, K] (rows may be strided): the
        activation pass, then the 4-bit GEMM, of this layer's number format,
        on one stream. Allocates qx, sx, xl1 and (unless y is given) Y."""
        if self.fmt == "int4":
            qx, sx, xl1 = _lib.quantize_act(x, self.inv_lambda, self.l1t, self.rank, stream)
            return _lib.w4a4_linear(qx, sx, xl1, self.qw, self.sw, self.l2t, self.bias, self.rank, act,
                                    out_dtype, y, stream)
        _lib._require(self.fmt == "mxfp4", f"unknown number format {self.fmt!r}")
        qx, sx, xl1 = _lib.quantize_act_mxfp4(x, self.inv_lambda, self.l1t, self.rank, stream)
        return _lib.mxfp4_linear(qx, sx, xl1, self.qw, self.sw, self.l2t, self.bias, self.rank, act,
                                 out_dtype, y, stream)


def awq_linear(x: torch.Tensor, layer: dict, y=None, stream=None) -> torch.Tensor:
    """Y = (x diag(inv_s)) deq(W) + bias for an AWQ W4A16 layer as
    quantize_awq() or load_awq_layer() return it (bias from the dict, if
    any): one GEMV launch. x bf16 [M, K] with M <= 16, contiguous."""
    return _lib.awq_gemv(x, layer.get("inv_s"), layer["qwt"], layer["scale_t"], layer["zero_t"], layer.get("bias"),
                         N=layer["N"], y=y, stream=stream)


class SvdqMLP:
    """fc1 (GELU) -> fc2 on M tokens, both INT4 or both MXFP4. ``forward(x)``
    copies x into the block's input buffer and runs the three launches;
    ``capture()`` records them once into a graph, after which ``replay(x)``
    does the same with one graph launch. Outputs land in ``self.y`` (bf16
    [M, fc2.N])."""

    def __init__(self, fc1: SvdqLinear, fc2: SvdqLinear, M: int):
        _lib._require(fc1.fmt == fc2.fmt and fc1.fmt in ("int4", "mxfp4"),
                      f"fc1 and fc2 must share a format (int4 or mxfp4), got {fc1.fmt} and {fc2.fmt}")
        _lib._require(fc2.K == fc1.N, f"fc2 takes K = {fc2.K}, fc1 gives N = {fc1.N}")
        _lib._require(fc1.N % 128 == 0, "fc1's N must be a multiple of 128 for the fused activation pass")
        _lib._require(fc2.rank <= 64, "fc2's rank must be at most 64 for the fused activation pass")
        self.fc1, self.fc2, self.M = fc1, fc2, M
        dev = fc1.qw.device
        K1, N1, N2 = fc1.K, fc1.N, fc2.N
        self.x = torch.empty((M, K1), dtype=torch.bfloat16, device=dev)
        self.mx = fc1.fmt == "mxfp4"
        sl, sdt = (8, torch.uint8) if self.mx else (4, torch.float16)
        self.qx1 = torch.empty((M, K1 // 2), dtype=torch.uint8, device=dev)
        self.sx1 = torch.empty(((K1 // 64 + 3) // 4, M, sl), dtype=sdt, device=dev)
        self.xl1_1 = torch.empty((M, fc1.rank), dtype=torch.float32, device=dev) if fc1.rank else None
        self.qx2 = torch.empty((M, N1 // 2), dtype=torch.uint8, device=dev)
        self.sx2 = torch.empty(((N1 // 64 + 3) // 4, M, sl), dtype=sdt, device=dev)
        self.xl1_2 = torch.empty((M, fc2.rank), dtype=torch.float32, device=dev) if fc2.rank else None
        nb = _lib.svdq_gemm_w4a4_quant_next_workspace_size(M, N1, fc2.rank)
        self.ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        self.ws_bytes = nb
        self.y = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
        self.graph = None

    def _launches(self):
        f1, f2, M = self.fc1, self.fc2, self.M
        act_pass = _lib.svdq_quantize_act_mxfp4 if self.mx else _lib.svdq_quantize_act
        fused = _lib.svdq_gemm_mxfp4_quant_next if self.mx else _lib.svdq_gemm_w4a4_quant_next
        gemm = _lib.svdq_gemm_mxfp4 if self.mx else _lib.svdq_gemm_w4a4
        act_pass(self.x, M, f1.K, f1.K, f1.inv_lambda, f1.l1t, f1.rank, self.qx1, self.sx1, self.xl1_1)
        fused(self.qx1, self.sx1, M, f1.K, f1.qw, f1.sw, f1.N, self.xl1_1, f1.l2t, f1.rank, f1.bias,
              _lib.ACT["gelu_tanh"], f2.inv_lambda, f2.l1t, f2.rank, self.qx2, self.sx2, self.xl1_2,
              self.ws if self.ws_bytes else None, self.ws_bytes)
        gemm(self.qx2, self.sx2, M, f2.K, f2.qw, f2.sw, f2.N, self.xl1_2, f2.l2t, f2.rank, f2.bias,
             _lib.ACT["none"], self.y, 0, f2.N)

    def _load(self, x):
        _lib._check_rows(x, "x", torch.bfloat16)
        _lib._require(tuple(x.shape) == tuple(self.x.shape), f"x must be {tuple(self.x.shape)}")
        if x.data_ptr() != self.x.data_ptr():
            self.x.copy_(x)

    def forward(self, x) -> torch.Tensor:
        self._load(x)
        self._launches()
        return self.y

    def capture(self, warmup: int = 1) -> CapturedSequence:
        self.graph = CapturedSequence(self._launches, warmup=warmup)
        return self.graph

    def replay(self, x=None) -> torch.Tensor:
        _lib._require(self.graph is not None, "capture() first")
        if x is not None:
            self._load(x)
        self.graph.replay()
        return self.y
