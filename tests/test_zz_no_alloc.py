"""The allocation-free entry point mmq_q4K_noalloc (q8_1 activations in the library's fixed
per-device scratch) against mmq_q4K (the same computation with a caller workspace): bit for
bit, on two calls in a row, the second with a smaller input, so that stale scratch contents
from the first call cannot leak into the second; plus the refusal of shapes beyond the
scratch, before anything is enqueued; and the entry point inside a captured HIP graph."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from quantized_prefill_gemm_amd import binding as B
from quantized_prefill_gemm_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_noalloc_matches_workspace_entry_twice():
    for M, N, K, seed in ((512, 4096, 4096, 61), (100, 300, 1280, 62)):      # second call smaller
        W, X = inputs.small_case("q4_K", M, N, K, seed=seed, gain=True)
        w = torch.from_numpy(W.reshape(-1)).to(DEV)
        x = torch.from_numpy(X).to(DEV)
        y_ref = B.mmq_q4K(w, x, N)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        assert B.mmq_q4K_noalloc(w, x, N, y) is y
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"{M}x{N}x{K}"


def test_noalloc_inside_a_captured_graph():
    """The use the entry point exists for: captured into a HIP graph (no allocation during
    capture), replayed three times with new activations copied in between, with eager work and
    synchronisation between the replays; every replay equals the eager mmq_q4K result."""
    M, N, K = 64, 1024, 2048
    W, _ = inputs.small_case("q4_K", M, N, K, seed=64)
    w = torch.from_numpy(W.reshape(-1)).to(DEV)
    x = torch.empty((M, K), dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    x.copy_(torch.from_numpy(inputs.small_case("q4_K", M, N, K, seed=65)[1]))
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up call outside the capture
        B.mmq_q4K_noalloc(w, x, N, y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.mmq_q4K_noalloc(w, x, N, y)
    for rep in range(3):
        X = inputs.small_case("q4_K", M, N, K, seed=66 + rep, gain=True)[1]
        x.copy_(torch.from_numpy(X))
        y.fill_(float("nan"))                       # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref = B.mmq_q4K(w, x, N)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"


def test_noalloc_largest_shape_and_refusal():
    # the largest q8_1 buffer the scratch holds: M * K * 1.125 <= 32 MiB
    M, N, K = 2048, 256, 11008
    assert B.q8_1_bytes(M, K) <= B.NOALLOC_SCRATCH_BYTES
    W, X = inputs.small_case("q4_K", M, N, K, seed=63)
    w = torch.from_numpy(W.reshape(-1)).to(DEV)
    x = torch.from_numpy(X).to(DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    B.mmq_q4K_noalloc(w, x, N, y)
    y_ref = B.mmq_q4K(w, x, N)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    # one more token row of K = 11008 than fits: refused, nothing enqueued (y untouched)
    M2 = B.NOALLOC_SCRATCH_BYTES // (K + 4 * (K // 32)) + 1
    assert B.q8_1_bytes(M2, K) > B.NOALLOC_SCRATCH_BYTES
    x2 = torch.zeros((M2, K), dtype=torch.float32, device=DEV)
    y2 = torch.full((M2, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(B.QPGError) as e:
        B.mmq_q4K_noalloc(w, x2, N, y2)
    assert e.value.status == B.QPG_ESCRATCH
    torch.cuda.synchronize()
    assert bool((y2 == 7.0).all())
