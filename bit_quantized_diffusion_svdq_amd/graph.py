"""Captured launch sequences: a run of library calls recorded once into a HIP
graph and replayed with no host launch work between the kernels.

Launch overhead between small kernels is what a compiled pipeline removes
(the donmalab.com page, section on squeezing out more performance: the same
Lite model went from 1.35x to 1.8x over BF16 once compiled; the remio.ai
page ties that gain to merged repeated graph operations). Here the kernels
are already fused per layer, so what is left is the host work between
launches; a transformer block's eight launches (activation pass + GEMM for
four linears) are recorded into one graph.

Plumbing only: the graph holds exactly the launches the callable issues
eagerly, with the same arguments. Every buffer the captured calls touch must
exist before capture and stay alive while the graph is used (pass outputs
with ``y=`` and use the raw entry points with preallocated qx / sx / xl1);
replays write into those same buffers. None of the library's calls
allocates or frees memory, synchronises, or issues a memset, so they are
capturable as they are.
"""
from __future__ import annotations

from typing import Callable

import torch


class CapturedSequence:
    """Record ``fn()`` (which issues library calls on the current stream)
    into one graph. ``replay()`` launches the graph on the current stream."""

    def __init__(self, fn: Callable[[], None], warmup: int = 1):
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):       # first-use host set-up stays outside the capture
                fn()
            with torch.cuda.graph(self.graph, stream=side):
                fn()
        torch.cuda.current_stream().wait_stream(side)

    def replay(self):
        self.graph.replay()
