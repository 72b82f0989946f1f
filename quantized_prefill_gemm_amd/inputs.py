"""Seeded synthetic inputs for the k-quant prefill GEMM (q4_K / q6_K weights, f32 activations).

This module only draws random numbers and places them at fixed byte offsets of the
weight blocks. It contains none of the method's arithmetic (no decoding, no
quantisation, no dot products), so the HIP path and the CPU oracle can both consume
its output without sharing any computation.

Block byte layouts (weights are stored row-major: row j of a [N x K] weight matrix is
K/256 consecutive blocks):

q4_K, 144 bytes per 256 weights
    +0   fp16  d       super-block scale
    +2   fp16  dmin    super-block min scale
    +4   12 B  packed eight 6-bit sub-block scales and eight 6-bit sub-block mins
    +16  128 B qs      4-bit quants, two per byte
  Only the 144-byte stride and "qs at +16" are fixed by the pages ("r28 - Direction-A
  raw-nibble NB kernel", sec. 3.2, B-side staging); the d / dmin / 12-byte placement is
  the GGUF q4_K layout. The 12 packed bytes hold exactly 16 six-bit fields that
  partition all 96 bits, so 12 independent uniform random bytes are the same thing as
  16 independent uniform 6-bit values (0..63) -- no packing code is needed here.

q6_K, 210 bytes per 256 weights
    +0   128 B ql      low 4 bits of the 6-bit quants
    +128 64 B  qh      high 2 bits of the 6-bit quants
    +192 16 B  sc      int8 sub-block scales (one per 16 weights)
    +208 fp16  d       super-block scale
  (GGUF q6_K layout; sizes and value ranges as in the 7B Q4_K_M-style workload.)

Distributions (the workloads of the pages, synthesised):
    q4_K: d, dmin = fp16(U[1e-3, 1e-2]); 6-bit scales/mins uniform 0..63; qs uniform bytes
    q6_K: ql, qh uniform bytes; sc uniform int8 in [-64, 63]; d = fp16(U[1e-3, 1e-2])
    activations: f32 N(0, 1), optionally row i scaled by a per-token gain g_i ~ U[0.5, 2]
"""
from __future__ import annotations

import numpy as np

QK_K = 256           # weights per super-block
Q4K_BLOCK = 144      # bytes per q4_K super-block
Q6K_BLOCK = 210      # bytes per q6_K super-block
QK8 = 32             # values per q8_1 block

BASE_SEED = 20260000


def _fp16_bytes(values: np.ndarray) -> np.ndarray:
    """Little-endian bytes of values rounded to IEEE binary16 (numpy's RNE cast)."""
    return values.astype(np.float16).view(np.uint8).reshape(values.shape + (2,))


def q4K_weights(N: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """uint8 array [N, (K/256)*144]: N rows of q4_K super-blocks."""
    if K % QK_K:
        raise ValueError("K must be a multiple of 256")
    nsb = K // QK_K
    blk = np.empty((N, nsb, Q4K_BLOCK), dtype=np.uint8)
    blk[:, :, 0:2] = _fp16_bytes(rng.uniform(1e-3, 1e-2, size=(N, nsb)))
    blk[:, :, 2:4] = _fp16_bytes(rng.uniform(1e-3, 1e-2, size=(N, nsb)))
    blk[:, :, 4:144] = rng.integers(0, 256, size=(N, nsb, 140), dtype=np.uint8)
    return blk.reshape(N, nsb * Q4K_BLOCK)


def q6K_weights(N: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """uint8 array [N, (K/256)*210]: N rows of q6_K super-blocks."""
    if K % QK_K:
        raise ValueError("K must be a multiple of 256")
    nsb = K // QK_K
    blk = np.empty((N, nsb, Q6K_BLOCK), dtype=np.uint8)
    blk[:, :, 0:192] = rng.integers(0, 256, size=(N, nsb, 192), dtype=np.uint8)
    blk[:, :, 192:208] = rng.integers(-64, 64, size=(N, nsb, 16)).astype(np.int8).view(np.uint8)
    blk[:, :, 208:210] = _fp16_bytes(rng.uniform(1e-3, 1e-2, size=(N, nsb)))
    return blk.reshape(N, nsb * Q6K_BLOCK)


def activations(M: int, K: int, rng: np.random.Generator, gain_rng: np.random.Generator | None = None) -> np.ndarray:
    """f32 [M, K] ~ N(0,1); with gain_rng, row i is multiplied by g_i ~ U[0.5, 2]."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    if gain_rng is not None:
        g = gain_rng.uniform(0.5, 2.0, size=(M, 1)).astype(np.float32)
        x = (x * g).astype(np.float32)
    return x


# The five workloads. Each entry: (weight type, M, N, K, per-token gain?)
CONFIGS = {
    1: ("q4_K", 64, 256, 256, False),        # tiny correctness case
    2: ("q4_K", 512, 4096, 4096, False),     # attention projection
    3: ("q4_K", 512, 11008, 4096, True),     # FFN gate/up, per-token gains
    4: ("q6_K", 512, 4096, 11008, False),    # attn_v / ffn_down
}

# 7B-style stack, one layer: (name, type, N, K); M = 1024 tokens, 32 layers.
STACK_LAYER = (
    ("q", "q4_K", 4096, 4096),
    ("k", "q4_K", 4096, 4096),
    ("v", "q6_K", 4096, 4096),
    ("o", "q4_K", 4096, 4096),
    ("gate", "q4_K", 11008, 4096),
    ("up", "q4_K", 11008, 4096),
    ("down", "q6_K", 4096, 11008),
)
STACK_LAYERS = 32
STACK_M = 1024


def _streams(entropy) -> tuple[np.random.Generator, np.random.Generator, np.random.Generator]:
    ss = np.random.SeedSequence(entropy)
    w_ss, x_ss, g_ss = ss.spawn(3)
    return np.random.default_rng(w_ss), np.random.default_rng(x_ss), np.random.default_rng(g_ss)


def make_config(cfg: int, n_rows: slice | None = None):
    """Return (wtype, M, N, K, W, X) for workload cfg in 1..4.

    The weight stream is drawn row-major, so any leading subset of rows is reproducible
    on its own only by drawing the whole matrix; n_rows selects rows after drawing.
    """
    wtype, M, N, K, gain = CONFIGS[cfg]
    w_rng, x_rng, g_rng = _streams(BASE_SEED + cfg)
    W = q4K_weights(N, K, w_rng) if wtype == "q4_K" else q6K_weights(N, K, w_rng)
    X = activations(M, K, x_rng, g_rng if gain else None)
    if n_rows is not None:
        W = W[n_rows]
    return wtype, M, N, K, W, X


def make_stack_matrix(layer: int, idx: int):
    """Weights of matrix idx (0..6, order of STACK_LAYER) of the given layer."""
    name, wtype, N, K = STACK_LAYER[idx]
    w_rng, _, _ = _streams([BASE_SEED + 5, layer, idx])
    W = q4K_weights(N, K, w_rng) if wtype == "q4_K" else q6K_weights(N, K, w_rng)
    return name, wtype, N, K, W


def make_stack_input(layer: int, idx: int, M: int = STACK_M):
    """f32 activation [M, K] fed to matrix idx of the given layer (fresh N(0,1) draw)."""
    _, _, _, K = STACK_LAYER[idx]
    _, x_rng, _ = _streams([BASE_SEED + 5, layer, idx])
    return activations(M, K, x_rng)


def small_case(wtype: str, M: int, N: int, K: int, seed: int, gain: bool = False):
    """Arbitrary-shape seeded case (tails, edge shapes) with the same distributions."""
    w_rng, x_rng, g_rng = _streams([BASE_SEED, seed, M, N, K])
    W = q4K_weights(N, K, w_rng) if wtype == "q4_K" else q6K_weights(N, K, w_rng)
    X = activations(M, K, x_rng, g_rng if gain else None)
    return W, X
