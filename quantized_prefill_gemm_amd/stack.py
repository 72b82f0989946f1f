"""The 7B-shaped prefill GEMM stack on one GPU: per layer the seven projections (q, k, v, o:
4096 x 4096; gate, up: 11008 x 4096; down: 4096 x 11008; q4_K except v and down, which are
q6_K), each fed by the q8_1 quantisation of its input. Orchestration only: every step is a
call into libqpg (quantize_q8_1, then the MMQ entry of the weight's form), in stream order,
so a pass can be launched eagerly or captured into one HIP graph (torch's graph API over the
library's own launches).

q, k and v read the same hidden state, gate and up the same normed state, so with quantize
sharing one quantize_q8_1 serves each group: 4 per layer instead of 7
(the prepass the pages run once per distinct activation, "31 - r28 - Direction-A raw-nibble
NB kernel", sec. 3.2).
"""
from __future__ import annotations

import torch

from . import binding as B
from .inputs import STACK_LAYER

# matrix position -> position whose input (and, with sharing, whose q8_1 buffer) it reads
SOURCE = {0: 0, 1: 0, 2: 0, 3: 3, 4: 4, 5: 4, 6: 6}
SOURCES = (0, 3, 4, 6)
MODES = ("all", "shared", "gemm")


class Stack:
    """Weights resident on the device, inputs / q8_1 buffers / outputs allocated once.

    weights[layer][idx]: raw q4_K / q6_K block buffers (uint8 device tensors) in the order of
    STACK_LAYER. q6: weight form of the q6_K matrices -- "raw" blocks, "prepared" or
    "expanded" (made here once, outside any pass). per_layer: every layer gets its own inputs
    and outputs (what a test compares); otherwise one input and one output per matrix
    position, reused by every layer (the layers then differ only in their weights, which is
    all the GEMM cost depends on).
    """

    def __init__(self, weights, M: int, q6: str = "expanded", per_layer: bool = False):
        if q6 not in ("raw", "prepared", "expanded"):
            raise ValueError(f"q6 form {q6!r}")
        self.M, self.q6, self.per_layer = M, q6, per_layer
        self.L = len(weights)
        dev = weights[0][0].device
        self.mats = []
        for layer in range(self.L):
            row = []
            for idx, (name, wtype, N, K) in enumerate(STACK_LAYER):
                w = weights[layer][idx]
                if wtype == "q6_K" and q6 == "prepared":
                    w = B.q6K_prepare(w, N, K)
                elif wtype == "q6_K" and q6 == "expanded":
                    w = B.q6K_expand(w, N, K)
                row.append(w)
            self.mats.append(row)
        nio = self.L if per_layer else 1
        self.x = [{src: torch.zeros((M, STACK_LAYER[src][3]), dtype=torch.float32, device=dev) for src in SOURCES}
                  for _ in range(nio)]
        self.xq = [[torch.empty(B.q8_1_bytes(M, K), dtype=torch.uint8, device=dev) for (_, _, _, K) in STACK_LAYER]
                   for _ in range(nio)]
        self.y = [[torch.empty((M, N), dtype=torch.float32, device=dev) for (_, _, N, _) in STACK_LAYER]
                  for _ in range(nio)]

    def io(self, layer: int) -> int:
        return layer if self.per_layer else 0

    def set_input(self, layer: int, src: int, x: torch.Tensor):
        """Input of the matrices reading position src (0: q/k/v, 3: o, 4: gate/up, 6: down)."""
        self.x[self.io(layer)][src].copy_(x)

    def output(self, layer: int, idx: int) -> torch.Tensor:
        return self.y[self.io(layer)][idx]

    def _gemm(self, layer: int, idx: int, xq: torch.Tensor, stream):
        _, wtype, N, K = STACK_LAYER[idx]
        w, y, M = self.mats[layer][idx], self.output(layer, idx), self.M
        if wtype == "q4_K":
            B.mmq_q4K_q8(w, xq, M, N, K, y, stream=stream)
        elif self.q6 == "prepared":
            B.mmq_q6K_prep_q8(w, xq, M, N, K, y, stream=stream)
        elif self.q6 == "expanded":
            B.mmq_q6K_exp_q8(w, xq, M, N, K, y, stream=stream)
        else:
            B.mmq_q6K_q8(w, xq, M, N, K, y, stream=stream)

    def run(self, mode: str = "shared", stream=None):
        """Enqueue one pass over all layers on `stream` (torch's current stream if None).
        all: a quantize_q8_1 before each of the 7 GEMMs of a layer; shared: one per distinct
        input (4 per layer); gemm: the shared pass without its quantizes (the GEMMs alone, on
        the q8_1 buffers a previous pass left)."""
        if mode not in MODES:
            raise ValueError(f"mode {mode!r}")
        for layer in range(self.L):
            io = self.io(layer)
            for idx in range(len(STACK_LAYER)):
                src = SOURCE[idx]
                if mode == "all":
                    B.quantize_q8_1(self.x[io][src], self.xq[io][idx], stream=stream)
                    self._gemm(layer, idx, self.xq[io][idx], stream)
                elif mode == "shared":
                    if src == idx:
                        B.quantize_q8_1(self.x[io][src], self.xq[io][src], stream=stream)
                    self._gemm(layer, idx, self.xq[io][src], stream)
                else:
                    self._gemm(layer, idx, self.xq[io][src], stream)

    def capture(self, mode: str = "shared") -> torch.cuda.CUDAGraph:
        """One pass captured as a graph: an eager pass on a side stream first (the library's
        first calls query the device), then the capture."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(mode)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(mode)
        return g

    def macs(self) -> int:
        return self.M * self.L * sum(N * K for _, _, N, K in STACK_LAYER)
