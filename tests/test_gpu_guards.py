"""Guard bands around every buffer a kernel writes.

Each output, workspace and repacked-weight buffer is a view into a larger allocation whose
4096 elements before and after it hold a sentinel pattern; after the call the guards must be
untouched (no kernel writes outside its buffer, at tile edges or in its tails) and every f32
output element must have been written (overwritten outputs: no sentinel left inside). Shapes
cover ragged M and N, N % 4 != 0 (the scalar epilogue), both q4_K token tiles, the three-group
split and the K split over workgroups.
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
GUARD = 4096
SENT32 = 0x7FBADBAD          # a NaN payload no kernel produces
SENT8 = 0xA5

SHAPES = [(1, 1, 256), (33, 130, 768), (64, 128, 256), (65, 257, 512), (100, 302, 1280),
          (16, 4096, 4096), (64, 4096, 2816), (300, 1000, 1536)]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Guarded:
    def __init__(self, n, dtype):
        self.n = n
        self.buf = torch.empty(n + 2 * GUARD, dtype=dtype, device=DEV)
        if dtype == torch.uint8:
            self.buf.fill_(SENT8)
        else:
            self.buf.view(torch.int32).fill_(SENT32)
        self.view = self.buf[GUARD:GUARD + n]

    def check(self, tag, filled=True):
        b = self.buf.view(torch.int32) if self.buf.dtype != torch.uint8 else self.buf
        s = SENT32 if self.buf.dtype != torch.uint8 else SENT8
        assert bool((b[:GUARD] == s).all()), f"{tag}: write before the buffer"
        assert bool((b[GUARD + self.n:] == s).all()), f"{tag}: write past the buffer"
        if filled and self.buf.dtype != torch.uint8:
            assert not bool((b[GUARD:GUARD + self.n] == s).any()), f"{tag}: output element not written"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_q4K_buffers_guarded(M, N, K):
    say(f"[guards q4_K {M}x{N}x{K}]")
    W, X = inputs.small_case("q4_K", M, N, K, seed=1400, gain=True)
    w = torch.from_numpy(W.reshape(-1)).to(DEV)
    x = torch.from_numpy(X).to(DEV)
    xq = Guarded(B.q8_1_bytes(M, K), torch.uint8)
    B.quantize_q8_1(x, xq.view)
    y = Guarded(M * N, torch.float32)
    B.mmq_q4K_q8(w, xq.view, M, N, K, y.view)
    s = Guarded(M * N * (K // 32), torch.int32)
    B.mmq_q4K_isums(w, xq.view, M, N, K, s.view)
    nws = B.mmq_sk_bytes(M, N, K, "q4K")
    ws = Guarded(max(nws // 4, 1), torch.float32)
    ysk = Guarded(M * N, torch.float32)
    B.mmq_q4K_q8_sk(w, xq.view, M, N, K, ysk.view, ws.view if nws else None)
    yf, xw = Guarded(M * N, torch.float32), Guarded(B.q8_1_bytes(M, K), torch.uint8)
    B.mmq_q4K(w, x, N, yf.view, xw.view)
    torch.cuda.synchronize()
    xq.check("q8_1 buffer", filled=False)
    y.check("mmq_q4K_q8 y")
    s.check("mmq_q4K_isums s")
    ysk.check("mmq_q4K_q8_sk y")
    if nws:
        ws.check("mmq_q4K_q8_sk workspace")
    yf.check("mmq_q4K y")
    xw.check("mmq_q4K workspace", filled=False)
    if B.q8_1_bytes(M, K) <= B.NOALLOC_SCRATCH_BYTES:
        yn = Guarded(M * N, torch.float32)
        B.mmq_q4K_noalloc(w, x, N, yn.view)
        torch.cuda.synchronize()
        yn.check("mmq_q4K_noalloc y")
        assert torch.equal(yn.view, y.view)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_q6K_buffers_guarded(M, N, K):
    say(f"[guards q6_K {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=1500, gain=True)
    w = torch.from_numpy(W.reshape(-1)).to(DEV)
    x = torch.from_numpy(X).to(DEV)
    xq = B.quantize_q8_1(x)
    wp = Guarded(B.q6K_prep_bytes(N, K), torch.uint8)
    B.q6K_prepare(w, N, K, wp.view)
    we = Guarded(B.q6K_exp_bytes(N, K), torch.uint8)
    B.q6K_expand(w, N, K, we.view)
    outs = {}
    for name, fn, wt in (("raw", B.mmq_q6K_q8, w), ("prepared", B.mmq_q6K_prep_q8, wp.view),
                         ("expanded", B.mmq_q6K_exp_q8, we.view)):
        outs[name] = Guarded(M * N, torch.float32)
        fn(wt, xq, M, N, K, outs[name].view)
    sk = {}
    for name, fn, wt, form in (("raw", B.mmq_q6K_q8_sk, w, "q6K"), ("prepared", B.mmq_q6K_prep_q8_sk, wp.view, "q6K_prep"),
                               ("expanded", B.mmq_q6K_exp_q8_sk, we.view, "q6K_exp")):
        nws = B.mmq_sk_bytes(M, N, K, form)
        ws = Guarded(max(nws // 4, 1), torch.float32)
        y = Guarded(M * N, torch.float32)
        fn(wt, xq, M, N, K, y.view, ws.view if nws else None)
        sk[name] = (y, ws, nws)
    s = Guarded(M * N * (K // 16), torch.int32)
    B.mmq_q6K_isums(w, xq, M, N, K, s.view)
    c = Guarded(M * N * (K // 32), torch.int32)
    B.mmq_q6K_exp_csums(we.view, xq, M, N, K, c.view)
    torch.cuda.synchronize()
    wp.check("q6K_prepare output", filled=False)
    we.check("q6K_expand output", filled=False)
    for name, g in outs.items():
        g.check(f"{name} y")
    for name, (y, ws, nws) in sk.items():
        y.check(f"{name} split-K y")
        if nws:
            ws.check(f"{name} split-K workspace")
    s.check("mmq_q6K_isums s")
    c.check("mmq_q6K_exp_csums s")
