"""The 32-layer 7B-shaped stack (M = 1024) through quantized_prefill_gemm_amd.stack -- the pass
bench.py times -- against the oracle.

One pass of all 32 layers with one quantize_q8_1 per distinct input (q/k/v and gate/up
share theirs) is captured as one HIP graph and replayed; every layer has its own inputs
and outputs. Layer 0: all seven GEMMs in full; layers 1..31: 16 sampled weight rows of
every GEMM (all 1024 tokens), the oracle regenerating those rows from the per-matrix seeds.
The eager pass with a quantize before each GEMM must give the same outputs bit for bit.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from oracle import oracle as O
from qblocks import tolerance_ok
from quantized_prefill_gemm_amd import inputs
from quantized_prefill_gemm_amd.stack import SOURCE, SOURCES, Stack

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
L, M = inputs.STACK_LAYERS, inputs.STACK_M
NMAT = len(inputs.STACK_LAYER)
SAMPLED_ROWS = 16


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def stack_run():
    rng = np.random.default_rng(2026)
    weights, host_w, rows = [], {}, {}
    for layer in range(L):
        row = []
        for idx in range(NMAT):
            name, wtype, N, K, W = inputs.make_stack_matrix(layer, idx)
            row.append(torch.from_numpy(W.reshape(-1)).to(DEV))
            if layer == 0:
                host_w[(layer, idx)] = W
            else:
                r = np.sort(rng.choice(N, SAMPLED_ROWS, replace=False))
                rows[(layer, idx)] = r
                host_w[(layer, idx)] = np.ascontiguousarray(W[r])
        weights.append(row)
        if layer % 8 == 7:
            say(f"  stack weights: {layer + 1}/{L} layers")
    st = Stack(weights, M, q6="expanded", per_layer=True)
    del weights
    host_x = {}
    for layer in range(L):
        for src in SOURCES:
            X = inputs.make_stack_input(layer, src)
            host_x[(layer, src)] = X
            st.set_input(layer, src, torch.from_numpy(X).to(DEV))
    say("  stack: capture (shared quantizes)")
    g = st.capture("shared")
    for rep in range(2):
        for layer in range(L):
            for idx in range(NMAT):
                st.output(layer, idx).fill_(float("nan"))      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
    return st, g, host_w, host_x, rows


def test_stack_layer0_all_gemms_full(stack_run):
    st, g, host_w, host_x, rows = stack_run
    for idx in range(NMAT):
        name, wtype, N, K = inputs.STACK_LAYER[idx]
        say(f"[stack layer 0 {name} {wtype} {M}x{N}x{K}, full]")
        got = st.output(0, idx).cpu().numpy()
        ref = O.mmq(wtype, host_w[(0, idx)], host_x[(0, SOURCE[idx])])
        ok, ratio, relmax = tolerance_ok(got, ref)
        say(f"  worst err/bound {ratio:.3e}, max rel err {relmax:.3e}")
        assert ok and relmax < 1e-4, f"layer 0 {name}"


def test_stack_layers_1_to_31_sampled_rows(stack_run):
    st, g, host_w, host_x, rows = stack_run
    worst = 0.0
    for layer in range(1, L):
        for idx in range(NMAT):
            name, wtype, N, K = inputs.STACK_LAYER[idx]
            r = rows[(layer, idx)]
            got = st.output(layer, idx)[:, torch.from_numpy(r).to(DEV)].cpu().numpy()
            ref = O.mmq(wtype, host_w[(layer, idx)], host_x[(layer, SOURCE[idx])])
            ok, ratio, relmax = tolerance_ok(got, ref)
            worst = max(worst, ratio)
            assert ok and relmax < 1e-4, f"layer {layer} {name}: err/bound {ratio}, rel {relmax}"
        if layer % 8 == 0:
            say(f"[stack layers 1..{layer} sampled rows: worst err/bound {worst:.3e}]")
    say(f"[stack layers 1..31 sampled rows: worst err/bound {worst:.3e}]")


def test_stack_eager_seven_quantizes_equals_shared_graph(stack_run):
    st, g, host_w, host_x, rows = stack_run
    say("[stack: eager pass with 7 quantizes per layer vs the shared-quantize graph]")
    ref = [[st.output(layer, idx).clone() for idx in range(NMAT)] for layer in range(L)]
    st.run("all")
    torch.cuda.synchronize()
    for layer in range(L):
        for idx in range(NMAT):
            assert torch.equal(st.output(layer, idx), ref[layer][idx]), f"layer {layer} {inputs.STACK_LAYER[idx][0]}"
    g.replay()
    torch.cuda.synchronize()
    for layer in range(L):
        for idx in range(NMAT):
            assert torch.equal(st.output(layer, idx), ref[layer][idx])
