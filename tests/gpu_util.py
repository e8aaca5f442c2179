"""Shared helpers for the GPU parity tests: moving oracle arrays to the
device in the library's layouts, and error measures."""
from __future__ import annotations

import sys

import numpy as np
import torch


def note(msg: str):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(dtype).cuda()


def dev_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float16))).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def host_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


class DevSvdq:
    """Oracle-prepared SVDQ layer moved to the device in the ABI layouts:
    L1 as [r][K] (transposed), L2 as [N][r] (transposed)."""

    def __init__(self, w):
        self.w = w
        self.rank = w.rank
        self.inv_lambda = dev(w.inv_lambda)
        self.l1t = dev_u16(np.ascontiguousarray(w.l1.T)) if w.rank else None
        self.l2t = dev_u16(np.ascontiguousarray(w.l2.T)) if w.rank else None
        self.qw = dev(w.qw)
        self.sw = dev_f16(w.sw)
        self.bias = dev_u16(w.bias) if w.bias is not None else None
