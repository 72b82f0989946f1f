"""Bit-exact witnesses at the kernel forms the launcher picks for the real workloads.

For every weight form the launcher has two tilings: a three-group split of each tile's
super-blocks when the grid has at most 256 tiles, else one tile per four-wave group (q4_K,
raw and prepared q6_K) or eight waves per tile (expanded q6_K). Every form is checked here
at >= 16 super-blocks, at the shapes the five workloads run:

1. Integer stage, in full: the isums / csums entry points (the same staging, unpack and
   MFMA source, compiled at the production launch bounds) at the workloads' own shapes and
   seeded data, every int32 sub-block / chunk sum against the oracle, compared in token
   slabs.
2. The production (folding) kernels themselves, bit for bit: inputs built so that every f32
   operation of the fold is exact -- q8_1 scales that are powers of two (each chunk holds one
   +-127 * 2^e and small multiples of 2^e, so d = 2^e and q is the chosen integer), weight
   scales d = 1, dmin = 1/2, small integer sub-block scales -- and bounded so that every
   partial sum is an integer multiple of the smallest term below 2^24 of it (the bound is
   asserted per test). The f32 result is then unique whatever the summation order, the
   oracle's fp64 result equals it, and a wrong integer sum, scale or token anywhere shows as a
   mismatch.
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from oracle import oracle as O
from qblocks import _Q4K_MAP
from quantized_prefill_gemm_amd import binding as B
from quantized_prefill_gemm_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def q4K_tile_m(M, N):
    """Token-tile height the q4_K launcher picks (mirror of the library's table): 32 when the
    64 x 128 grid has <= 128 tiles, or M <= 256 and more than 256 tiles; else 64."""
    t64 = -(-M // 64) * -(-N // 128)
    return 32 if (t64 <= 128 or (M <= 256 and t64 > 256)) else 64


def launch_form(kind, M, N, K, pieces=1):
    """The tiling the launcher picks (mirrors the launch code): 'split3' = three groups over
    each tile's super-blocks (<= 256 tiles), 'one-group' / 'eight-wave' otherwise; q4_K forms
    carry the token-tile height ('/tm32' for 32-token tiles)."""
    tn = 64 if kind == "exp" else 128
    tm = q4K_tile_m(M, N) if kind == "q4K" else 64
    tiles = -(-M // tm) * -(-N // tn)
    if tiles * pieces <= 256 and (K // 256) // pieces >= 3:
        form = "split3"
    else:
        form = "eight-wave" if kind == "exp" else "one-group"
    return form + ("/tm32" if tm == 32 else "")


def quantized(X):
    xq = B.quantize_q8_1(dev(X))
    q, _, _ = O.quantize_q8_1(X)
    return xq, q


def compare_slabs(got: torch.Tensor, ref_fn, M: int, slab: int, tag: str):
    """got: device int32 [M][N][n]; ref_fn(t0, t1) -> oracle int32 [t1-t0][N][n]."""
    for t0 in range(0, M, slab):
        t1 = min(M, t0 + slab)
        g = got[t0:t1].cpu().numpy()
        r = ref_fn(t0, t1)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{tag}: {len(bad)} mismatching sums in tokens {t0}..{t1 - 1}, "
                                 f"first at {bad[:3].tolist()}")


# --------------------------------------------------------------------------- 1. integer stage

def config_or_stack(src):
    if src[0] == "cfg":
        wtype, M, N, K, W, X = inputs.make_config(src[1])
        return wtype, M, N, K, W, X
    _, idx = src
    name, wtype, N, K, W = inputs.make_stack_matrix(0, idx)
    X = inputs.make_stack_input(0, idx)
    return wtype, X.shape[0], N, K, W, X


ISUM_CASES = [
    # (label, data source, weight form, expected tiling)
    ("cfg2 q4_K 512x4096x4096", ("cfg", 2), "q4K", "split3"),
    ("cfg3 q4_K 512x11008x4096", ("cfg", 3), "q4K", "one-group"),
    ("cfg4 q6_K raw 512x4096x11008", ("cfg", 4), "raw", "split3"),
    ("cfg4 q6_K prepared 512x4096x11008", ("cfg", 4), "prep", "split3"),
    ("cfg4 q6_K expanded 512x4096x11008", ("cfg", 4), "exp", "eight-wave"),
    ("stack q q4_K 1024x4096x4096", ("stack", 0), "q4K", "one-group"),
    ("stack gate q4_K 1024x11008x4096", ("stack", 4), "q4K", "one-group"),
    ("stack v q6_K raw 1024x4096x4096", ("stack", 2), "raw", "one-group"),
    ("stack v q6_K prepared 1024x4096x4096", ("stack", 2), "prep", "one-group"),
    ("stack v q6_K expanded 1024x4096x4096", ("stack", 2), "exp", "eight-wave"),
    ("stack down q6_K raw 1024x4096x11008", ("stack", 6), "raw", "one-group"),
    ("stack down q6_K prepared 1024x4096x11008", ("stack", 6), "prep", "one-group"),
    ("stack down q6_K expanded 1024x4096x11008", ("stack", 6), "exp", "eight-wave"),
]


def short_prompt(M, N, K, seed):
    """The workload's distributions (per-token gains) at a short prompt length."""
    W, X = inputs.small_case("q4_K", M, N, K, seed=seed, gain=True)
    return "q4_K", M, N, K, W, X


SHORT_CASES = [
    # 32-token q4_K tiles: three-group split (few tiles) and one group per tile (> 256 tiles)
    ("q4_K 16x4096x4096", (16, 4096, 4096), "split3/tm32"),
    ("q4_K 128x4096x4096", (128, 4096, 4096), "split3/tm32"),
    ("q4_K 256x11008x4096", (256, 11008, 4096), "one-group/tm32"),
]


@pytest.mark.parametrize("label,shape,tiling", SHORT_CASES, ids=[c[0] for c in SHORT_CASES])
def test_integer_stage_full_short_prompts(label, shape, tiling):
    wtype, M, N, K, W, X = short_prompt(*shape, seed=71)
    assert launch_form("q4K", M, N, K) == tiling
    say(f"[integer stage {label}: {tiling}]")
    xq, q = quantized(X)
    s = B.mmq_q4K_isums(dev(W.reshape(-1)), xq, M, N, K)
    torch.cuda.synchronize()
    compare_slabs(s, lambda t0, t1: O.isums(wtype, W, q[t0:t1]), M, 64, label)


@pytest.mark.parametrize("label,src,form,tiling", ISUM_CASES, ids=[c[0] for c in ISUM_CASES])
def test_integer_stage_full_at_workload_shapes(label, src, form, tiling):
    wtype, M, N, K, W, X = config_or_stack(src)
    assert launch_form(form, M, N, K) == tiling, "the case no longer exercises the tiling it names"
    say(f"[integer stage {label}: {tiling}, {K // 256} super-blocks]")
    xq, q = quantized(X)
    w = dev(W.reshape(-1))
    if form == "q4K":
        s = B.mmq_q4K_isums(w, xq, M, N, K)
    elif form == "raw":
        s = B.mmq_q6K_isums(w, xq, M, N, K)
    elif form == "prep":
        s = B.mmq_q6K_prep_isums(B.q6K_prepare(w, N, K), xq, M, N, K)
    else:
        s = B.mmq_q6K_exp_csums(B.q6K_expand(w, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    del w, xq
    if form == "exp":
        ref = lambda t0, t1: O.q6K_chunk_sums(W, q[t0:t1])
        slab = 16
    else:
        ref = lambda t0, t1: O.isums(wtype, W, q[t0:t1])
        slab = 64 if wtype == "q4_K" else 32
    compare_slabs(s, ref, M, slab, label)


def test_integer_stage_expanded_split_form():
    """Expanded q6_K with at most 256 tiles of 64 x 64 (512 x 2048 x 11008, 43 super-blocks):
    the three-group form, on the first 2048 rows of the down-projection workload."""
    wtype, M, N, K, W, X = inputs.make_config(4)
    W = np.ascontiguousarray(W[:2048])
    N = 2048
    assert launch_form("exp", M, N, K) == "split3"
    say("[integer stage expanded q6_K 512x2048x11008: split3]")
    xq, q = quantized(X)
    s = B.mmq_q6K_exp_csums(B.q6K_expand(dev(W.reshape(-1)), N, K), xq, M, N, K)
    torch.cuda.synchronize()
    compare_slabs(s, lambda t0, t1: O.q6K_chunk_sums(W, q[t0:t1]), M, 32, "exp split3")


def test_prepared_isums_config4_against_oracle():
    """Prepared q6_K integer sums on the first 256 rows of the down-projection workload, all
    tokens and super-blocks, against the oracle (not against the raw-block kernel)."""
    wtype, M, N, K, W, X = inputs.make_config(4)
    Wr = np.ascontiguousarray(W[:256])
    say("[prepared q6_K isums cfg4 rows 0..255]")
    xq, q = quantized(X)
    s = B.mmq_q6K_prep_isums(B.q6K_prepare(dev(Wr.reshape(-1)), 256, K), xq, M, 256, K)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), O.isums("q6_K", Wr, q))


# --------------------------------------------------------------------------- 2. exact production outputs

def exact_activations(M, K, rng, vmax, emin, emax):
    """f32 [M][K]: chunk c of token i is 2^e_ic * v with v integers in [-vmax, vmax] and one
    position forced to +-127, so that q8_1 gives d = 2^e exactly (amax = 127 * 2^e), 1/d = 2^-e
    and q = v. Returns (X, v, e)."""
    nc = K // 32
    v = rng.integers(-vmax, vmax + 1, size=(M, nc, 32))
    pos = rng.integers(0, 32, size=(M, nc))
    sign = rng.choice([-127, 127], size=(M, nc))
    np.put_along_axis(v, pos[..., None], sign[..., None], axis=2)
    e = rng.integers(emin, emax + 1, size=(M, nc))
    X = (v * np.exp2(e)[..., None]).astype(np.float32).reshape(M, K)
    return X, v.reshape(M, K), e


def check_quantizer_exactness(X, v, e):
    q, dh, ss = O.quantize_q8_1(X)
    assert np.array_equal(q, v.astype(np.int8))
    assert np.array_equal(dh, np.exp2(e).astype(np.float16).view(np.uint16))


def q4K_small_scale_weights(N, K, rng):
    """q4_K blocks with d = 1, dmin = 1/2, every 6-bit scale and min in [0, 3], random nibbles.
    The 12 packed bytes are assembled from the fields through the bit-destination table of
    the block format (the same table as the test-side encoder)."""
    nsb = K // 256
    blk = np.zeros((N, nsb, 144), np.uint8)
    blk[:, :, 0:2] = np.array([1.0], np.float16).view(np.uint8)
    blk[:, :, 2:4] = np.array([0.5], np.float16).view(np.uint8)
    sc = rng.integers(0, 4, size=(N, nsb, 8))
    m = rng.integers(0, 4, size=(N, nsb, 8))
    packed = np.zeros((N, nsb, 12), np.uint8)
    for (field, s, bit), (byte, dst) in _Q4K_MAP.items():
        val = (sc if field == "sc" else m)[:, :, s]
        packed[:, :, byte] |= (((val >> bit) & 1) << dst).astype(np.uint8)
    blk[:, :, 4:16] = packed
    blk[:, :, 16:] = rng.integers(0, 256, size=(N, nsb, 128), dtype=np.uint8)
    return blk.reshape(N, nsb * 144)


def q6K_small_scale_weights(N, K, rng):
    """q6_K blocks with d = 1, int8 scales in [-2, 2], random 6-bit values."""
    nsb = K // 256
    blk = np.empty((N, nsb, 210), np.uint8)
    blk[:, :, :192] = rng.integers(0, 256, size=(N, nsb, 192), dtype=np.uint8)
    blk[:, :, 192:208] = rng.integers(-2, 3, size=(N, nsb, 16)).astype(np.int8).view(np.uint8)
    blk[:, :, 208:210] = np.array([1.0], np.float16).view(np.uint8)
    return blk.reshape(N, nsb * 210)


def exactness_bound(wtype, v, e, emin):
    """Largest, over tokens, of the sum of |every fold term| in units of 2^emin (the smallest
    term granularity), from worst-case weights: q4_K |sc * nib| <= 3 * 15 and min terms
    |dmin * m * ssum| <= 1/2 * 3 * 32 * max|q| per sub-block; q6_K |sc * (q6 - 32)| <= 2 * 32.
    Below 2^24 every partial sum of every order is exact in f32."""
    da = np.exp2(e - emin)                                     # [M][nc], integers
    absq = np.abs(v).reshape(v.shape[0], -1, 32).sum(axis=2)   # [M][nc] sum |q| per chunk
    if wtype == "q4_K":
        scale_terms = (da * absq * 3 * 15).sum(axis=1)
        min_terms = (da * absq * 3 * 0.5).sum(axis=1)
        return float(np.max(scale_terms + min_terms))
    return float(np.max((da * absq * 2 * 32).sum(axis=1)))


EXACT_CASES = [
    # (label, form, M, N, K, expected tiling, split-K pieces or None for the plain entry)
    ("q4_K 512x11008x4096", "q4K", 512, 11008, 4096, "one-group", None),
    ("q4_K 512x4096x4096", "q4K", 512, 4096, 4096, "split3", None),
    ("q4_K 1024x11008x4096", "q4K", 1024, 11008, 4096, "one-group", None),
    ("q4_K K-split 512x512x4096", "q4K", 512, 512, 4096, "split3/tm32", 4),
    ("q4_K 512x1376x4096", "q4K", 512, 1376, 4096, "split3/tm32", None),
    ("q4_K 128x4096x4096", "q4K", 128, 4096, 4096, "split3/tm32", None),
    ("q4_K 256x11008x4096", "q4K", 256, 11008, 4096, "one-group/tm32", None),
    ("q4_K K-split 16x4096x4096", "q4K", 16, 4096, 4096, "one-group/tm32", 8),
    ("q4_K K-split 64x4096x4096", "q4K", 64, 4096, 4096, "split3/tm32", 4),
    ("q6_K raw 512x4096x11008", "raw", 512, 4096, 11008, "split3", None),
    ("q6_K raw 1024x4096x11008", "raw", 1024, 4096, 11008, "one-group", None),
    ("q6_K prepared 512x4096x11008", "prep", 512, 4096, 11008, "split3", None),
    ("q6_K prepared 1024x4096x11008", "prep", 1024, 4096, 11008, "one-group", None),
    ("q6_K expanded 512x4096x11008", "exp", 512, 4096, 11008, "eight-wave", None),
    ("q6_K expanded 512x2048x11008", "exp", 512, 2048, 11008, "split3", None),
    ("q6_K expanded K-split 512x512x11008", "exp", 512, 512, 11008, "split3", 4),
]


@pytest.mark.parametrize("label,form,M,N,K,tiling,pieces", EXACT_CASES, ids=[c[0] for c in EXACT_CASES])
def test_production_kernels_bit_exact_on_exact_inputs(label, form, M, N, K, tiling, pieces):
    wtype = "q4_K" if form == "q4K" else "q6_K"
    sk_form = {"q4K": "q4K", "raw": "q6K", "prep": "q6K_prep", "exp": "q6K_exp"}[form]
    if pieces:
        assert B.mmq_sk_bytes(M, N, K, sk_form) == pieces * M * N * 4
    assert launch_form(form, M, N, K, pieces or 1) == tiling
    say(f"[exact production {label}: {tiling}{f', {pieces} pieces' if pieces else ''}]")
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    vmax, emin, emax = (15, -1, 0) if wtype == "q4_K" else (7, -1, 0)
    X, v, e = exact_activations(M, K, rng, vmax, emin, emax)
    check_quantizer_exactness(X, v, e)
    bound = exactness_bound(wtype, v, e, emin)
    assert bound < 2 ** 24, f"inputs not exact-safe: {bound}"
    W = q4K_small_scale_weights(N, K, rng) if wtype == "q4_K" else q6K_small_scale_weights(N, K, rng)
    xq = B.quantize_q8_1(dev(X))
    w = dev(W.reshape(-1))
    if form == "prep":
        w = B.q6K_prepare(w, N, K)
    elif form == "exp":
        w = B.q6K_expand(w, N, K)
    if pieces:
        fn = {"q4K": B.mmq_q4K_q8_sk, "q6K": B.mmq_q6K_q8_sk, "q6K_prep": B.mmq_q6K_prep_q8_sk,
              "q6K_exp": B.mmq_q6K_exp_q8_sk}[sk_form]
        y = fn(w, xq, M, N, K)
    else:
        fn = {"q4K": B.mmq_q4K_q8, "raw": B.mmq_q6K_q8, "prep": B.mmq_q6K_prep_q8, "exp": B.mmq_q6K_exp_q8}[form]
        y = fn(w, xq, M, N, K)
    torch.cuda.synchronize()
    g = y.cpu().numpy().astype(np.float64)
    r = O.mmq(wtype, W, X)
    assert np.array_equal(r.astype(np.float32).astype(np.float64), r), "oracle result not an f32 value"
    if not np.array_equal(g, r):
        bad = np.argwhere(g != r)
        i, j = bad[0]
        raise AssertionError(f"{label}: {len(bad)} outputs differ, first ({i}, {j}): {g[i, j]!r} vs {r[i, j]!r}")
