"""Seeded synthetic inputs for the SVDQuant W4A4 linear and the AWQ W4A16 GEMV.

This module is shared by the CPU oracle, the tests and the benchmark. It only
draws random numbers and rounds them to bf16 storage; it holds none of the
method's arithmetic (no smoothing, no SVD, no quantisation).

Workloads stand in for the diffusion-transformer layers that the Nunchaku /
SVDQuant pages benchmark (ERNIE-Image-Turbo and FLUX at 1024x1024): the pages
name no public dataset and ship no weights, so activations and weights are
Gaussian with planted outlier channels, which is the structure the pages blame
for the difficulty of 4-bit quantisation ("SVDQuant moves hard values out of
4-bit" section of the remio.ai page; "core challenge" section of the
donmalab.com page).

Draw order per layer, from ``numpy.random.default_rng(seed)``:
X ~ N(0, 1) [M, K] -> outlier column indices (without replacement) -> those
columns of X multiplied by the outlier factor -> W ~ N(0, std_w) [K, N] ->
bias ~ N(0, 0.02) [N] -> (AWQ only) per-input-channel scale ~ U(0.5, 2) [K].
Every float is rounded to bf16 (round to nearest even) before use.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    K: int
    N: int
    rank: int = 32
    group: int = 64
    alpha: float = 0.5
    n_outliers: int = 0
    outlier_factor: float = 1.0
    std_w: float = 0.02
    act: str = "none"          # "none" or "gelu_tanh"
    seed: int = 0
    kind: str = "svdq"         # "svdq" or "awq"
    note: str = ""


# Sizes of the workloads (token count M = 4096 image tokens at 1024^2, plus
# 512 text tokens for the MLP pair; hidden 3072 as in FLUX/ERNIE-class DiTs).
CONFIGS = {
    "tiny": LayerConfig("tiny", M=256, K=512, N=512, rank=16, n_outliers=4,
                        outlier_factor=20.0, note="tiny SVDQ W4A4 linear"),
    "qkv": LayerConfig("qkv", M=4096, K=3072, N=9216, rank=32, n_outliers=31,
                       outlier_factor=30.0, note="DiT attention QKV projection"),
    "mlp_fc1": LayerConfig("mlp_fc1", M=4608, K=3072, N=12288, rank=32, n_outliers=31,
                           outlier_factor=30.0, act="gelu_tanh",
                           note="DiT MLP fc1 with GELU(tanh) epilogue"),
    "mlp_fc2": LayerConfig("mlp_fc2", M=4608, K=12288, N=3072, rank=32,
                           note="DiT MLP fc2 (input is fc1's bf16 GELU output)"),
    "awq": LayerConfig("awq", M=4, K=3072, N=18432, kind="awq",
                       note="AWQ W4A16 adaLN modulation GEMV"),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 storage (RTNE); returns uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray            # uint16 bf16 bits [M, K]
    w: np.ndarray            # uint16 bf16 bits [K, N]
    bias: np.ndarray         # uint16 bf16 bits [N]
    outlier_cols: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    chan_scale: np.ndarray | None = None   # float32 [K] (AWQ per-channel scale)


def make_layer(cfg: LayerConfig, M: int | None = None, seed: int | None = None) -> LayerInputs:
    """Draw one layer's inputs. ``M`` overrides the token count (same weights
    distribution, fewer rows) for reduced-size tests."""
    M = cfg.M if M is None else M
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    x = rng.standard_normal((M, cfg.K), dtype=np.float32)
    cols = np.zeros(0, np.int64)
    if cfg.n_outliers:
        cols = np.sort(rng.choice(cfg.K, cfg.n_outliers, replace=False))
        x[:, cols] *= np.float32(cfg.outlier_factor)
    w = (rng.standard_normal((cfg.K, cfg.N), dtype=np.float32) * np.float32(cfg.std_w))
    bias = rng.standard_normal(cfg.N, dtype=np.float32) * np.float32(0.02)
    chan = None
    if cfg.kind == "awq":
        chan = rng.uniform(0.5, 2.0, cfg.K).astype(np.float32)
    return LayerInputs(cfg, bf16_round(x), bf16_round(w), bf16_round(bias), cols, chan)


def make_matrix_bf16(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    """Generic seeded Gaussian matrix as bf16 bits (used for edge-case shapes)."""
    rng = np.random.default_rng(seed)
    return bf16_round(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std))


def make_codes(rows: int, cols: int, seed: int, lo: int, hi: int) -> np.ndarray:
    """Seeded integer codes in [lo, hi] (int8), for operand-level kernel tests."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols), dtype=np.int64).astype(np.int8)


def make_f16_scales(rows: int, cols: int, seed: int, lo: float, hi: float) -> np.ndarray:
    """Seeded positive scales stored as fp16 bit patterns (uint16)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=(rows, cols)).astype(np.float16).view(np.uint16)
