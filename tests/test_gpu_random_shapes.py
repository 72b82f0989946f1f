"""Seeded random shapes through every MMQ entry point, against the oracle.

The other parity tests pick their shapes by hand (tails, tile edges, the workloads); this one
draws them: M in [1, 300], N in [1, 700], K in 256 * [1, 14] (and six larger draws up to
1100 x 4500 x 3072), so ragged tiles, odd and even
super-block counts, N % 4 != 0 (the scalar epilogue) and both q4_K token-tile heights turn up
in combinations nobody chose. For each shape: the q4_K and q6_K products on every weight form
(raw blocks, prepared, expanded; plain and K-split entry points), outputs within the method's
tolerance, and the integer sums of the raw q4_K / q6_K kernels bit for bit. The raw q6_K
blocks sit at an address 2 mod 4 in every other case.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from oracle import oracle as O
from qblocks import tolerance_ok
from quantized_prefill_gemm_amd import binding as B
from quantized_prefill_gemm_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
N_CASES = 20
N_LARGE = 6


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def shapes():
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(N_CASES):
        M = int(rng.integers(1, 301))
        N = int(rng.integers(1, 701))
        K = 256 * int(rng.integers(1, 15))
        out.append((i, M, N, K))
    return out


def large_shapes():
    """Fewer, larger draws (M 257..1100, N 1000..4500, K to 3072): grids past 256 tiles, where the
    launchers take one tile per four-wave group (eight waves for expanded q6_K), with ragged
    tails and long K, and the 32-token q4_K tiles of large grids (M <= 256)."""
    rng = np.random.default_rng(20261203)
    out = []
    while len(out) < N_LARGE:
        M, N, K = int(rng.integers(257, 1101)), int(rng.integers(1000, 4501)), 256 * int(rng.integers(1, 13))
        if M * N * K <= 12e9:                       # keeps the oracle's share of the suite short
            out.append((N_CASES + len(out), M, N, K))
    return out


def isums_checked(M, N, K):
    """Integer sums are compared in full up to 2^26 of them (the witness tests cover the
    integer stage of the large workloads in token slabs)."""
    return M * N * (K // 16) <= (1 << 26)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_at(a, shift):
    b = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    buf = torch.zeros(b.size + 256, dtype=torch.uint8, device=DEV)
    v = buf[shift:shift + b.size]
    v.copy_(torch.from_numpy(b))
    return v


def check(g, r, tag):
    ok, ratio, relmax = tolerance_ok(g, r)
    assert ok and relmax < 1e-4, f"{tag}: err/bound {ratio:.3e}, rel {relmax:.3e}"
    return ratio


@pytest.mark.parametrize("i,M,N,K", shapes() + large_shapes())
def test_random_shape_q4K(i, M, N, K):
    say(f"[random q4_K case {i}: {M}x{N}x{K}]")
    W, X = inputs.small_case("q4_K", M, N, K, seed=700 + i, gain=True)
    xq = B.quantize_q8_1(dev(X))
    w = dev(W.reshape(-1))
    y = B.mmq_q4K_q8(w, xq, M, N, K)
    ysk = B.mmq_q4K_q8_sk(w, xq, M, N, K)
    s = B.mmq_q4K_isums(w, xq, M, N, K) if isums_checked(M, N, K) else None
    torch.cuda.synchronize()
    q, _, _ = O.quantize_q8_1(X)
    if s is not None:
        assert np.array_equal(s.cpu().numpy(), O.isums("q4_K", W, q))
    r = O.mmq("q4_K", W, X)
    worst = max(check(y.cpu().numpy(), r, "q8 entry"), check(ysk.cpu().numpy(), r, "split-K entry"))
    say(f"  worst err/bound {worst:.3e}")


@pytest.mark.parametrize("i,M,N,K", shapes() + large_shapes())
def test_random_shape_q6K_all_forms(i, M, N, K):
    say(f"[random q6_K case {i}: {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=900 + i, gain=True)
    xq = B.quantize_q8_1(dev(X))
    w = dev_at(W, 2) if i % 2 else dev(W.reshape(-1))
    outs = {"raw": B.mmq_q6K_q8(w, xq, M, N, K), "raw split-K": B.mmq_q6K_q8_sk(w, xq, M, N, K)}
    s = B.mmq_q6K_isums(w, xq, M, N, K) if isums_checked(M, N, K) else None
    wp = B.q6K_prepare(dev(W.reshape(-1)), N, K)          # the repack wants 4-byte blocks
    outs["prepared"] = B.mmq_q6K_prep_q8(wp, xq, M, N, K)
    outs["prepared split-K"] = B.mmq_q6K_prep_q8_sk(wp, xq, M, N, K)
    we = B.q6K_expand(w, N, K)
    outs["expanded"] = B.mmq_q6K_exp_q8(we, xq, M, N, K)
    outs["expanded split-K"] = B.mmq_q6K_exp_q8_sk(we, xq, M, N, K)
    torch.cuda.synchronize()
    q, _, _ = O.quantize_q8_1(X)
    if s is not None:
        assert np.array_equal(s.cpu().numpy(), O.isums("q6_K", W, q))
    r = O.mmq("q6_K", W, X)
    worst = max(check(y.cpu().numpy(), r, form) for form, y in outs.items())
    say(f"  {len(outs)} forms, worst err/bound {worst:.3e}")
