"""Concurrent calls on two streams share no hidden state.

Every entry point except mmq_q4K_noalloc works only on the caller's buffers, so calls running at
the same time on different streams (each with its own outputs and K-split workspace) must give
exactly the outputs they give one after another. Four products -- q4_K and raw q6_K through
the plain entry points, expanded q6_K and q4_K through the K-split ones -- are issued three
times, alternating between two streams of default priority with no synchronisation between
them, and compared bit for bit with the sequential results.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from quantized_prefill_gemm_amd import binding as B
from quantized_prefill_gemm_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_concurrent_streams_match_sequential():
    cases = []
    for i, (wtype, form, M, N, K) in enumerate([("q4_K", "q4K", 256, 2048, 2048), ("q6_K", "q6K", 130, 1024, 2816),
                                                ("q6_K", "q6K_exp_sk", 32, 1024, 2816), ("q4_K", "q4K_sk", 32, 1024, 4096)]):
        W, X = inputs.small_case(wtype, M, N, K, seed=1300 + i, gain=True)
        w = torch.from_numpy(W.reshape(-1)).to(DEV)
        if form == "q6K_exp_sk":
            w = B.q6K_expand(w, N, K)
        xq = B.quantize_q8_1(torch.from_numpy(X).to(DEV))
        nws = B.mmq_sk_bytes(M, N, K, form[:-3]) if form.endswith("_sk") else 0
        ws = torch.empty(max(nws // 4, 1), dtype=torch.float32, device=DEV) if nws else None
        cases.append((form, w, xq, M, N, K, ws))
    torch.cuda.synchronize()

    def call(case, y, stream=None):
        form, w, xq, M, N, K, ws = case
        if form == "q4K":
            return B.mmq_q4K_q8(w, xq, M, N, K, y, stream=stream)
        if form == "q6K":
            return B.mmq_q6K_q8(w, xq, M, N, K, y, stream=stream)
        if form == "q6K_exp_sk":
            return B.mmq_q6K_exp_q8_sk(w, xq, M, N, K, y, ws, stream=stream)
        return B.mmq_q4K_q8_sk(w, xq, M, N, K, y, ws, stream=stream)

    refs = []
    for c in cases:
        y = torch.empty((c[3], c[4]), dtype=torch.float32, device=DEV)
        call(c, y)
        refs.append(y)
    torch.cuda.synchronize()
    say(f"[streams: {len(cases)} products, sequential reference done]")

    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    for rep in range(3):
        outs = [torch.full((c[3], c[4]), float("nan"), dtype=torch.float32, device=DEV) for c in cases]
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            call(c, outs[i], stream=streams[(i + rep) % 2])
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            assert torch.equal(outs[i], refs[i]), f"repeat {rep}, {c[0]} {c[3]}x{c[4]}x{c[5]}"
    say("[streams: three concurrent repeats equal to the sequential results]")
