"""Fused projections: one SVDQ layer for several projections that read the
same activations (the query, key and value projections of an attention
block), and how its packed tensors map back to the separate modules.

Some optimised implementations merge the query, key and value projections
into one grouped operation, and a loader then has to know the tensor order
and how the grouped parameters map to the individual modules (remio.ai page,
section on the generic integration path and its overhead). This library's
convention:

  * Order. The fused layer's output columns are the projections one after
    another along N, in the order given (for attention: [Q | K | V]).
    Projection i owns columns [off_i, off_i + n_i), off_i = n_0 + ... + n_{i-1}.
  * What is shared. The activation side (smoothing vector inv_lambda, the
    down-projection L1, and so qx, sx and xl1) belongs to the fused layer:
    the offline preparation runs on the concatenated weight [W_0 | W_1 | ...]
    (one smoothing vector, one SVD), so one activation pass serves all the
    projections. The fused layer is therefore not the same as separately
    prepared layers, and separately packed layers cannot be concatenated
    into it.
  * What is per column. Everything on the weight side is indexed by output
    column and slices along N: codes qw [N][K/2] (rows), INT4 scales
    [ceil(G/4)][N][4] and MXFP4 exponents [ceil(K/256)][N][8] (middle axis),
    the up-projection L2 stored as [N][r] (rows) and the bias [N]. A slice
    of the fused layer's weight side, used with the fused layer's qx, sx and
    xl1, gives exactly the slice of the fused output (each output column is
    computed on its own).
  * Sizes. Each n_i must be a multiple of 8 (the GEMM's N rule); the fused
    output is [M][sum n_i] and split_columns returns strided views of it.

These helpers only index and copy tensors; no arithmetic of the layer runs
here.
"""
from __future__ import annotations

from typing import Sequence

import torch


def column_offsets(sizes: Sequence[int]) -> list[int]:
    """Start column of each projection (and the total at the end)."""
    offs = [0]
    for n in sizes:
        if n <= 0 or n % 8:
            raise ValueError(f"projection widths must be positive multiples of 8, got {n}")
        offs.append(offs[-1] + int(n))
    return offs


def split_columns(y: torch.Tensor, sizes: Sequence[int]) -> list[torch.Tensor]:
    """Views of the fused output y [M, sum(sizes)] (or a row-strided output
    with that many columns), one per projection, in order."""
    offs = column_offsets(sizes)
    if y.shape[-1] != offs[-1]:
        raise ValueError(f"output has {y.shape[-1]} columns, the projections {offs[-1]}")
    return [y[..., offs[i]:offs[i + 1]] for i in range(len(sizes))]


def column_slice(qw: torch.Tensor, sw: torch.Tensor, l2t, bias, n0: int, n1: int):
    """Weight side of output columns [n0, n1) of a packed layer (INT4 or
    MXFP4), as contiguous tensors: (qw [n][K/2], sw [quads][n][4 or 8],
    l2t [n][r] or None, bias [n] or None)."""
    N = qw.shape[0]
    if not (0 <= n0 < n1 <= N) or n0 % 8 or (n1 - n0) % 8:
        raise ValueError(f"column range [{n0}, {n1}) must lie in [0, {N}) on multiples of 8")
    if sw.dim() != 3 or sw.shape[1] != N:
        raise ValueError("scales must be in the quad-major layout [quads][N][4 or 8]")
    return (qw[n0:n1].contiguous(), sw[:, n0:n1, :].contiguous(),
            None if l2t is None else l2t[n0:n1].contiguous(),
            None if bias is None else bias[n0:n1].contiguous())


def projection_weights(qw, sw, l2t, bias, sizes: Sequence[int]):
    """column_slice for every projection of a fused layer, in order."""
    offs = column_offsets(sizes)
    if offs[-1] != qw.shape[0]:
        raise ValueError(f"layer has {qw.shape[0]} output columns, the projections {offs[-1]}")
    return [column_slice(qw, sw, l2t, bias, offs[i], offs[i + 1]) for i in range(len(sizes))]
