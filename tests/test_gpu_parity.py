"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (from the method's stated targets):
  * q8_1 output (int8 values, fp16 scale bits, int16 block sums): bit-exact.
  * integer sub-block sums (isums entry points): bit-exact.
  * f32 outputs: |gpu - oracle| <= 1e-4*|oracle| + 1e-3*rms(oracle) element-wise, the
    oracle being exact up to fp64 summation.
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from oracle import oracle as O
from qblocks import tolerance_ok, encode_q4K, encode_q6K, near_tie_blocks
from quantized_prefill_gemm_amd import binding as B
from quantized_prefill_gemm_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def parse_q8(buf: torch.Tensor, M: int, K: int):
    b = buf.cpu().numpy()
    q = b[:M * K].view(np.int8).reshape(M, K)
    hdr = b[M * K:M * K + 4 * M * (K // 32)].view(np.uint32).reshape(M, K // 32)
    dh = (hdr & 0xFFFF).astype(np.uint16)
    ss = (hdr >> 16).astype(np.uint16).view(np.int16)
    return q, dh, ss


def gpu_quantize(x: np.ndarray):
    M, K = x.shape
    xq = B.quantize_q8_1(dev(x))
    torch.cuda.synchronize()
    return xq, parse_q8(xq, M, K)


def assert_q8_equal(x: np.ndarray, tag: str):
    _, (q, dh, ss) = gpu_quantize(x)
    rq, rdh, rss = O.quantize_q8_1(x)
    assert np.array_equal(q, rq), f"{tag}: q mismatch at {np.argwhere(q != rq)[:5]}"
    assert np.array_equal(dh, rdh), f"{tag}: fp16 scale mismatch"
    assert np.array_equal(ss, rss), f"{tag}: block sum mismatch"


# ----------------------------------------------------------------------------- q8_1

@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_quantize_bitexact_configs(cfg):
    say(f"[quantize cfg{cfg}]")
    _, M, N, K, _, X = inputs.make_config(cfg)
    assert_q8_equal(X, f"cfg{cfg}")


def test_quantize_edge_cases():
    say("[quantize edges]")
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "q8_1_ties.json")))
    rng = np.random.default_rng(9)
    cases = {
        "zeros": np.zeros((3, 256), np.float32),
        "ties": np.tile(np.array(g["x"], np.float32), (2, 8)),
        "tiny": (rng.standard_normal((4, 256)) * 1e-30).astype(np.float32),
        "subnormal_scale": (rng.standard_normal((4, 256)) * 1e-39).astype(np.float32),
        "huge": (rng.standard_normal((4, 256)) * 3e4).astype(np.float32),
        "outlier": np.where(rng.random((8, 512)) < 0.01, 900.0, rng.standard_normal((8, 512)) * 0.1).astype(np.float32),
        "k32": rng.standard_normal((7, 32)).astype(np.float32),
        "k96": rng.standard_normal((5, 96)).astype(np.float32),
        "m1": rng.standard_normal((1, 4096)).astype(np.float32),
        "ramp": (np.arange(64 * 256, dtype=np.float32).reshape(64, 256) % 97 - 48.5) / 7,
    }
    for tag, x in cases.items():
        assert_q8_equal(x, tag)


@pytest.mark.parametrize("amax", [127.0, 63.5, 127.0 * 2.0 ** -20])
def test_quantize_near_ties(amax):
    say(f"[quantize near ties, amax {amax}]")
    x = near_tie_blocks(amax)
    b = x.reshape(-1, 32)
    live = np.any(b != 0, axis=1)                    # the rest are zero blocks filling the rows
    assert (b[live, 0] == np.float32(amax)).all() and live.sum() == 58
    assert_q8_equal(x, f"near ties, amax {amax}")


# ----------------------------------------------------------------------------- integer stage

def gpu_isums(wtype, W, xq, M, N, K):
    fn = B.mmq_q4K_isums if wtype == "q4_K" else B.mmq_q6K_isums
    s = fn(dev(W.reshape(-1)), xq, M, N, K)
    torch.cuda.synchronize()
    return s.cpu().numpy()


ISUM_SHAPES = [(64, 256, 256), (1, 1, 256), (33, 130, 512), (65, 257, 768), (128, 384, 1024), (7, 129, 2816)]


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("M,N,K", ISUM_SHAPES)
def test_isums_bitexact(wtype, M, N, K):
    say(f"[isums {wtype} {M}x{N}x{K}]")
    W, X = inputs.small_case(wtype, M, N, K, seed=3)
    xq, (q, _, _) = gpu_quantize(X)
    s = gpu_isums(wtype, W, xq, M, N, K)
    ref = O.isums(wtype, W, q)
    assert np.array_equal(s, ref), f"mismatches: {np.count_nonzero(s != ref)}"


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_isums_bitexact_config_rows(cfg):
    """Integer sums of the real workloads on a slice of weight rows (all tokens, all K)."""
    wtype, M, N, K, W, X = inputs.make_config(cfg)
    rows = slice(0, min(N, 256))
    Wr = np.ascontiguousarray(W[rows])
    n = Wr.shape[0]
    say(f"[isums cfg{cfg} rows {n}]")
    xq, (q, _, _) = gpu_quantize(X)
    s = gpu_isums(wtype, Wr, xq, M, n, K)
    assert np.array_equal(s, O.isums(wtype, Wr, q))


# ----------------------------------------------------------------------------- outputs

def gpu_mmq(wtype, W, X, N):
    fn = B.mmq_q4K if wtype == "q4_K" else B.mmq_q6K
    y = fn(dev(W.reshape(-1)), dev(X), N)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_out(g, r, tag):
    ok, ratio, relmax = tolerance_ok(g, r)
    say(f"  {tag}: worst err/bound {ratio:.3e}, max rel err (|r|>=rms) {relmax:.3e}")
    assert ok, f"{tag}: err/bound {ratio}"
    assert relmax < 1e-4, f"{tag}: relative error {relmax}"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_mmq_configs_full(cfg):
    wtype, M, N, K, W, X = inputs.make_config(cfg)
    say(f"[mmq cfg{cfg} {wtype} {M}x{N}x{K}]")
    g = gpu_mmq(wtype, W, X, N)
    r = O.mmq(wtype, W, X)
    check_out(g, r, f"cfg{cfg}")


TAIL_SHAPES = [(1, 1, 256), (1, 130, 512), (33, 1, 256), (33, 130, 768), (65, 257, 512), (100, 300, 1280),
               (64, 128, 256), (63, 127, 4096)]


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_mmq_tails(wtype, M, N, K):
    say(f"[mmq tail {wtype} {M}x{N}x{K}]")
    W, X = inputs.small_case(wtype, M, N, K, seed=5, gain=True)
    check_out(gpu_mmq(wtype, W, X, N), O.mmq(wtype, W, X), f"{wtype} {M}x{N}x{K}")


def dev_at(a: np.ndarray, shift: int) -> torch.Tensor:
    """The bytes of a on the device, starting `shift` bytes past a 256-byte boundary (a view
    into a larger buffer)."""
    b = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    buf = torch.zeros(b.size + 256, dtype=torch.uint8, device=DEV)
    v = buf[shift:shift + b.size]
    v.copy_(torch.from_numpy(b))
    return v


@pytest.mark.parametrize("shift", [2, 6])
@pytest.mark.parametrize("M,N,K", [(33, 130, 768), (100, 200, 1024), (65, 257, 2816), (512, 130, 11008)])
def test_q6K_raw_blocks_at_two_byte_alignment(M, N, K, shift):
    """Raw q6_K blocks at an address that is 2 mod 4 (the blocks' own alignment, their fp16 d):
    integer sums bit-exact against the oracle, outputs within the tolerance, through the q8,
    f32 and K-split entry points; every row start is then 2 mod 4 (K/256 even) or alternates
    (K/256 odd)."""
    say(f"[q6_K raw blocks at +{shift}: {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=21 + shift, gain=True)
    w = dev_at(W, shift)
    assert w.data_ptr() % 4 == 2
    xq, (q, _, _) = gpu_quantize(X)
    s = B.mmq_q6K_isums(w, xq, M, N, K)
    y = B.mmq_q6K_q8(w, xq, M, N, K)
    yf = B.mmq_q6K(w, dev(X), N)
    ysk = B.mmq_q6K_q8_sk(w, xq, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), O.isums("q6_K", W, q))
    r = O.mmq("q6_K", W, X)
    check_out(y.cpu().numpy(), r, f"q8 entry +{shift}")
    assert torch.equal(yf, y)
    check_out(ysk.cpu().numpy(), r, f"split-K entry +{shift}")
    # the same blocks 16-byte aligned give the same outputs bit for bit
    y16 = B.mmq_q6K_q8(dev(W.reshape(-1)), xq, M, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y16, y)


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
def test_f32_entry_equals_quantize_then_q8(wtype):
    M, N, K = 96, 200, 1024
    say(f"[f32 entry == q8 entry {wtype}]")
    W, X = inputs.small_case(wtype, M, N, K, seed=6)
    y1 = gpu_mmq(wtype, W, X, N)
    xq = B.quantize_q8_1(dev(X))
    fn = B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8
    y2 = fn(dev(W.reshape(-1)), xq, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2.cpu().numpy())


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
def test_metamorphic(wtype):
    """Y(2^t X) = 2^t Y(X) bit for bit; Y(-X) = -Y(X) to a few ulp (the q4_K min term is
    accumulated by the matrix core, whose f32 rounding is scale-invariant but not
    sign-symmetric); the integer sums of -X are exactly the negated sums."""
    M, N, K = 64, 256, 2048
    say(f"[metamorphic {wtype}]")
    W, X = inputs.small_case(wtype, M, N, K, seed=7)
    y = gpu_mmq(wtype, W, X, N)
    for t in (-4, 3):
        assert np.array_equal(gpu_mmq(wtype, W, X * np.float32(2.0 ** t), N), y * np.float32(2.0 ** t))
    yn = gpu_mmq(wtype, W, -X, N)
    rms = float(np.sqrt(np.mean(y.astype(np.float64) ** 2)))
    assert np.max(np.abs(yn.astype(np.float64) + y)) <= 2.0 ** -20 * rms
    xq_p, _ = gpu_quantize(X)
    xq_n, _ = gpu_quantize(-X)
    assert np.array_equal(gpu_isums(wtype, W, xq_n, M, N, K), -gpu_isums(wtype, W, xq_p, M, N, K))


# ----------------------------------------------------------------------------- prepared q6_K

def gpu_prepare(W, N, K):
    wp = B.q6K_prepare(dev(W.reshape(-1)), N, K)
    torch.cuda.synchronize()
    return wp


@pytest.mark.parametrize("M,N,K", ISUM_SHAPES)
def test_q6K_prep_isums_bitexact(M, N, K):
    say(f"[q6_K prepared isums {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=3)
    xq, (q, _, _) = gpu_quantize(X)
    s = B.mmq_q6K_prep_isums(gpu_prepare(W, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), O.isums("q6_K", W, q))


@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_q6K_prep_tails(M, N, K):
    say(f"[q6_K prepared mmq {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=5, gain=True)
    xq, _ = gpu_quantize(X)
    y = B.mmq_q6K_prep_q8(gpu_prepare(W, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq("q6_K", W, X), f"prep {M}x{N}x{K}")


def test_q6K_prep_config4_full():
    wtype, M, N, K, W, X = inputs.make_config(4)
    say(f"[q6_K prepared cfg4 {M}x{N}x{K}]")
    xq, _ = gpu_quantize(X)
    wp = gpu_prepare(W, N, K)
    y = B.mmq_q6K_prep_q8(wp, xq, M, N, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq(wtype, W, X), "prep cfg4")
    rows = slice(0, 256)
    Wr = np.ascontiguousarray(W[rows])
    s = B.mmq_q6K_prep_isums(gpu_prepare(Wr, 256, K), xq, M, 256, K)
    torch.cuda.synchronize()
    q, _, _ = O.quantize_q8_1(X)
    assert np.array_equal(s.cpu().numpy(), O.isums(wtype, Wr, q))


# ----------------------------------------------------------------------------- expanded q6_K

def gpu_expand(W, N, K):
    we = B.q6K_expand(dev(W.reshape(-1)), N, K)
    torch.cuda.synchronize()
    return we


@pytest.mark.parametrize("M,N,K", ISUM_SHAPES)
def test_q6K_exp_csums_bitexact(M, N, K):
    say(f"[q6_K expanded csums {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=3)
    xq, (q, _, _) = gpu_quantize(X)
    s = B.mmq_q6K_exp_csums(gpu_expand(W, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    ref = O.q6K_chunk_sums(W, q)
    got = s.cpu().numpy()
    assert np.array_equal(got, ref), f"mismatches: {np.count_nonzero(got != ref)}"


@pytest.mark.parametrize("M,N,K", TAIL_SHAPES)
def test_q6K_exp_tails(M, N, K):
    say(f"[q6_K expanded mmq {M}x{N}x{K}]")
    W, X = inputs.small_case("q6_K", M, N, K, seed=5, gain=True)
    xq, _ = gpu_quantize(X)
    y = B.mmq_q6K_exp_q8(gpu_expand(W, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq("q6_K", W, X), f"exp {M}x{N}x{K}")


def test_q6K_exp_config4_full():
    wtype, M, N, K, W, X = inputs.make_config(4)
    say(f"[q6_K expanded cfg4 {M}x{N}x{K}]")
    xq, (q, _, _) = gpu_quantize(X)
    y = B.mmq_q6K_exp_q8(gpu_expand(W, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq(wtype, W, X), "exp cfg4")
    rows = slice(0, 192)
    Wr = np.ascontiguousarray(W[rows])
    s = B.mmq_q6K_exp_csums(gpu_expand(Wr, 192, K), xq, M, 192, K)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), O.q6K_chunk_sums(Wr, q))


# ----------------------------------------------------------------------------- K split over workgroups

SK_FORMS = ["q4K", "q6K", "q6K_prep", "q6K_exp"]
SK_SHAPES = [(1, 1, 1536), (64, 100, 1536), (33, 130, 2816), (100, 300, 4096), (130, 257, 11008)]
BPB = {"q4_K": 144, "q6_K": 210}


def sk_operands(form, W, N, K):
    if form == "q6K_prep":
        return gpu_prepare(W, N, K)
    if form == "q6K_exp":
        return gpu_expand(W, N, K)
    return dev(W.reshape(-1))


def sk_call(form, w, xq, M, N, K, y=None, ws=None):
    fn = {"q4K": B.mmq_q4K_q8_sk, "q6K": B.mmq_q6K_q8_sk, "q6K_prep": B.mmq_q6K_prep_q8_sk,
          "q6K_exp": B.mmq_q6K_exp_q8_sk}[form]
    return fn(w, xq, M, N, K, y=y, ws=ws)


def plain_call(form, w, xq, M, N, K):
    fn = {"q4K": B.mmq_q4K_q8, "q6K": B.mmq_q6K_q8, "q6K_prep": B.mmq_q6K_prep_q8,
          "q6K_exp": B.mmq_q6K_exp_q8}[form]
    return fn(w, xq, M, N, K)


@pytest.mark.parametrize("form", SK_FORMS)
@pytest.mark.parametrize("M,N,K", SK_SHAPES)
def test_splitk_matches_oracle(form, M, N, K):
    """K split over P workgroups: y against the oracle; plane p of the workspace against the
    oracle on super-blocks [p*nsb/P, (p+1)*nsb/P) alone; y is the piece-order f32 sum of the
    planes, bit for bit, and the same on a second call."""
    wtype = "q4_K" if form == "q4K" else "q6_K"
    nws = B.mmq_sk_bytes(M, N, K, form)
    P = nws // (4 * M * N)
    say(f"[split-K {form} {M}x{N}x{K} pieces {P}]")
    assert P >= 2 and nws == P * M * N * 4
    W, X = inputs.small_case(wtype, M, N, K, seed=9, gain=True)
    xq, _ = gpu_quantize(X)
    w = sk_operands(form, W, N, K)
    ws = torch.full((nws // 4,), float("nan"), dtype=torch.float32, device=DEV)
    y1 = sk_call(form, w, xq, M, N, K, ws=ws)
    torch.cuda.synchronize()
    planes = ws.view(P, M, N).cpu().numpy()
    y2 = sk_call(form, w, xq, M, N, K, ws=ws)
    torch.cuda.synchronize()
    g = y1.cpu().numpy()
    assert np.array_equal(g, y2.cpu().numpy())
    check_out(g, O.mmq(wtype, W, X), f"sk {form} {M}x{N}x{K}")
    acc = planes[0].copy()
    for p in range(1, P):
        acc = acc + planes[p]
    assert np.array_equal(acc, g)
    nsb = K // 256
    Wb = W.reshape(N, nsb, BPB[wtype])
    for p in range(P):
        b0, b1 = p * nsb // P, (p + 1) * nsb // P
        Wp = np.ascontiguousarray(Wb[:, b0:b1]).reshape(N, -1)
        rp = O.mmq(wtype, Wp, np.ascontiguousarray(X[:, 256 * b0:256 * b1]))
        check_out(planes[p], rp, f"  piece {p} (super-blocks {b0}..{b1 - 1})")


@pytest.mark.parametrize("form", SK_FORMS)
def test_splitk_without_split_is_the_plain_entry(form):
    """Shapes that need no split (many tiles, too few super-blocks for two pieces of three
    with several token-tile rows, or one super-block) take no workspace and give the plain
    entry point's output bit for bit."""
    wtype = "q4_K" if form == "q4K" else "q6_K"
    for M, N, K in ((100, 100, 1280), (640, 2100, 1024), (16, 100, 256)):
        assert B.mmq_sk_bytes(M, N, K, form) == 0
        say(f"[split-K no split {form} {M}x{N}x{K}]")
        W, X = inputs.small_case(wtype, M, N, K, seed=10)
        xq, _ = gpu_quantize(X)
        w = sk_operands(form, W, N, K)
        y = sk_call(form, w, xq, M, N, K)
        y0 = plain_call(form, w, xq, M, N, K)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), y0.cpu().numpy())


@pytest.mark.parametrize("form,N,K", [("q4K", 1376, 4096), ("q4K", 512, 4096), ("q6K", 512, 11008),
                                      ("q6K_prep", 512, 11008), ("q6K_exp", 512, 11008)])
def test_splitk_shard_shapes(form, N, K):
    """One GPU's share of a 7B-style layer split eight ways along N (M = 512 prompt tokens),
    the shapes the split is for: full output against the oracle."""
    wtype = "q4_K" if form == "q4K" else "q6_K"
    M = 512
    say(f"[split-K shard {form} {M}x{N}x{K} pieces {B.mmq_sk_bytes(M, N, K, form) // (4 * M * N)}]")
    W, X = inputs.small_case(wtype, M, N, K, seed=11, gain=True)
    xq, _ = gpu_quantize(X)
    y = sk_call(form, sk_operands(form, W, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq(wtype, W, X), f"shard {form}")


# ----------------------------------------------------------------------------- maximum sizes

KMAX_RAW = 1 << 24                    # K <= 2^24 (per-tile byte offsets stay below 2^31)
KMAX_PREP = (1 << 24) - 256           # prepared: (K/256) * 32 KiB < 2^31
KMAX_EXP = 61230 * 256                # expanded: (K/256) * 35,072 < 2^31


def big_activations(K, rows, src_rows, seed):
    """Device X [len(src_rows)][K] whose token t is host row src_rows[t] of `rows` distinct
    seeded rows (the oracle needs only those)."""
    _, Xd = inputs.small_case("q4_K", rows, 1, K, seed=seed, gain=True)
    idx = torch.tensor(src_rows, dtype=torch.int64, device=DEV)
    return Xd, dev(Xd).index_select(0, idx)


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
def test_max_K_and_q_plane_past_2GiB(wtype):
    """K = 2^24 (65,536 super-blocks) with M = 150 tokens and N = 5 rows: the q8_1 plane is
    2.5 GB, so tokens 128.. start past 2^31 bytes. Each token is one of 4 distinct rows: its
    output must match the oracle on that row, and equal tokens must agree bit for bit. The
    K-split entry point (3 tiles, 8 pieces) is checked the same way."""
    M, N, K = 150, 5, KMAX_RAW
    src = [(7 * t) % 4 for t in range(M)]
    say(f"[max K {wtype} {M}x{N}x{K}]")
    Xh, Xd = big_activations(K, 4, src, seed=21)
    Wh, _ = inputs.small_case(wtype, 1, N, K, seed=22)
    w = dev(Wh.reshape(-1))
    xq = B.quantize_q8_1(Xd)
    plain = B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8
    sk = B.mmq_q4K_q8_sk if wtype == "q4_K" else B.mmq_q6K_q8_sk
    y = plain(w, xq, M, N, K)
    ys = sk(w, xq, M, N, K)
    torch.cuda.synchronize()
    del Xd, xq
    ref = O.mmq(wtype, Wh, Xh)                      # [4][N]
    for tag, g in (("plain", y.cpu().numpy()), ("split", ys.cpu().numpy())):
        for r in range(4):
            toks = [t for t in range(M) if src[t] == r]
            assert all(np.array_equal(g[toks[0]], g[t]) for t in toks)
        check_out(g, ref[src], f"max K {wtype} {tag}")


@pytest.mark.parametrize("form", ["q6K_prep", "q6K_exp"])
def test_max_K_prepared_and_expanded(form):
    """The largest K each repacked q6_K layout accepts (its per-tile record range just under
    2^31 bytes), M = 3, N = 5."""
    K = KMAX_PREP if form == "q6K_prep" else KMAX_EXP
    M, N = 3, 5
    say(f"[max K {form} {M}x{N}x{K}]")
    Wh, Xh = inputs.small_case("q6_K", M, N, K, seed=23, gain=True)
    w = dev(Wh.reshape(-1))
    xq = B.quantize_q8_1(dev(Xh))
    if form == "q6K_prep":
        assert B.q6K_prep_bytes(N, K + 256) == 0
        y = B.mmq_q6K_prep_q8(B.q6K_prepare(w, N, K), xq, M, N, K)
    else:
        assert B.q6K_exp_bytes(N, K + 256) == 0
        y = B.mmq_q6K_exp_q8(B.q6K_expand(w, N, K), xq, M, N, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq("q6_K", Wh, Xh), f"max K {form}")


def test_degenerate_zero_blocks():
    """Zero activations (amax = 0: d = 0, q = 0, ssum = 0), all-zero tokens, zero weight
    super-blocks (d = dmin = 0) and zero scales: exact zeros where the definition gives zero,
    the oracle elsewhere, for every weight form."""
    M, N, K = 70, 130, 1024
    say("[degenerate zero blocks]")
    for wtype in ("q4_K", "q6_K"):
        W, X = inputs.small_case(wtype, M, N, K, seed=24, gain=True)
        X = X.copy()
        X[5] = 0.0                                   # a whole token of zeros
        X[9, 64:96] = 0.0                            # one zero chunk
        X[:, 512:544] = 0.0                          # a zero chunk in every token
        W = W.copy()
        bpb = 144 if wtype == "q4_K" else 210
        Wb = W.reshape(N, K // 256, bpb)
        Wb[3, :, :] = 0                              # a whole row of zero blocks
        Wb[17, 2, :] = 0                             # one zero super-block
        W = Wb.reshape(N, -1)
        r = O.mmq(wtype, W, X)
        assert np.all(r[5] == 0) and np.all(r[:, 3] == 0)
        xq, _ = gpu_quantize(X)
        w = dev(W.reshape(-1))
        outs = [("raw", (B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8)(w, xq, M, N, K))]
        if wtype == "q6_K":
            outs.append(("prep", B.mmq_q6K_prep_q8(B.q6K_prepare(w, N, K), xq, M, N, K)))
            outs.append(("exp", B.mmq_q6K_exp_q8(B.q6K_expand(w, N, K), xq, M, N, K)))
        torch.cuda.synchronize()
        for tag, y in outs:
            g = y.cpu().numpy()
            assert np.all(g[5] == 0) and np.all(g[:, 3] == 0), f"{wtype} {tag}"
            check_out(g, r, f"zeros {wtype} {tag}")


def test_closed_form_scale_path_on_gpu():
    """All nib = 1, sc = 1, d = 1, X = 1: Y = K * 0.99993896484375 exactly (golden)."""
    K = 1024
    w = np.tile(encode_q4K(1.0, 0.0, [1] * 8, [0] * 8, [1] * 256), (130, K // 256))
    y = gpu_mmq("q4_K", w, np.ones((70, K), np.float32), 130)
    assert np.all(y == np.float32(1023.9375))


@pytest.mark.parametrize("layer", [0, 31])
def test_stack_layers(layer):
    """7B-style stack (M = 1024), each of the 4 distinct GEMM shapes of a layer (q4_K q and
    gate, q6_K v and down; q6_K also on expanded weights, the form the stack bench runs):
    layer 0 against the oracle in full, layer 31 on 16 sampled weight rows."""
    rng = np.random.default_rng(17 + layer)
    for idx in (0, 2, 4, 6):               # q (q4_K 4096^2), v (q6_K 4096^2), gate, down
        name, wtype, N, K, W = inputs.make_stack_matrix(layer, idx)
        X = inputs.make_stack_input(layer, idx)
        say(f"[stack layer {layer} {name} {wtype} {X.shape[0]}x{N}x{K}]")
        outs = [("", gpu_mmq(wtype, W, X, N))]
        if wtype == "q6_K":
            xq, _ = gpu_quantize(X)
            y = B.mmq_q6K_exp_q8(gpu_expand(W, N, K), xq, X.shape[0], N, K)
            torch.cuda.synchronize()
            outs.append((" expanded", y.cpu().numpy()))
        rows = np.arange(N) if layer == 0 else np.sort(rng.choice(N, 16, replace=False))
        r = O.mmq(wtype, W if layer == 0 else W[rows], X)
        for tag, g in outs:
            check_out(g[:, rows], r, f"stack L{layer} {name}{tag}")


def test_graph_replay_matches_eager():
    """A small two-layer stack (quantize + q4_K / q6_K / prepared / expanded q6_K GEMMs, one with
    the K split) captured as one
    graph: every replay, with eager work and synchronisations between replays, must give
    the eager outputs bit for bit."""
    M = 96
    specs = [("q4_K", 384, 512), ("q6_K", 256, 768), ("q6p", 200, 1024), ("q4_K", 130, 768), ("q6x", 190, 768),
             ("q4s", 200, 3072)]
    mats, xs, xqs, ys = [], [], [], []
    ws = torch.empty(B.mmq_sk_bytes(M, 200, 3072, "q4K") // 4, dtype=torch.float32, device=DEV)
    assert ws.numel() > 0
    for i, (kind, N, K) in enumerate(specs):
        wtype = "q4_K" if kind in ("q4_K", "q4s") else "q6_K"
        W, X = inputs.small_case(wtype, M, N, K, seed=40 + i)
        w = dev(W.reshape(-1))
        if kind == "q6p":
            w = B.q6K_prepare(w, N, K)
        elif kind == "q6x":
            w = B.q6K_expand(w, N, K)
        mats.append((kind, N, K, w))
        xs.append(dev(X))
        xqs.append(torch.empty(B.q8_1_bytes(M, K), dtype=torch.uint8, device=DEV))
        ys.append(torch.empty((M, N), dtype=torch.float32, device=DEV))

    def run():
        for (kind, N, K, w), x, xq, y in zip(mats, xs, xqs, ys):
            B.quantize_q8_1(x, xq)
            if kind == "q4_K":
                B.mmq_q4K_q8(w, xq, M, N, K, y)
            elif kind == "q6_K":
                B.mmq_q6K_q8(w, xq, M, N, K, y)
            elif kind == "q6p":
                B.mmq_q6K_prep_q8(w, xq, M, N, K, y)
            elif kind == "q4s":
                B.mmq_q4K_q8_sk(w, xq, M, N, K, y, ws)
            else:
                B.mmq_q6K_exp_q8(w, xq, M, N, K, y)

    say("[graph replay]")
    run()
    torch.cuda.synchronize()
    ref = [y.cpu().numpy().copy() for y in ys]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        run()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            assert np.array_equal(y.cpu().numpy(), ref[i]), f"replay {rep}, GEMM {i}"



def test_calib_mfma_peak_runs():
    # the measurement helper of bench.py: every workgroup reports a positive tick count
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(B.LIB_PATH), "libqpg_calib.so"))
    lib.qpg_calib_mfma_i8.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.qpg_calib_mfma_i8.restype = ctypes.c_int
    out = torch.zeros(256 * 4, dtype=torch.int64, device="cuda:0")
    assert lib.qpg_calib_mfma_i8(256, 200, ctypes.c_void_p(out.data_ptr()), None) == 0
    torch.cuda.synchronize()
    v = out.view(256, 4).cpu().numpy()
    assert (v[:, 0] > 0).all() and (v[:, 1] > 0).all() and (v[:, 3] == 0).all()


def test_extreme_magnitudes():
    """Integer sums at their largest magnitudes (|I| = 15*127*32 for q4_K, |J| = 32*127*16
    for q6_K, the range the 1.5*2^23 accumulator constant has to hold): every nibble 15 /
    every q6 value -32 or +31, extreme scales, activations of +-1 (q = +-127)."""
    say("[extreme magnitudes]")
    K = 512
    X = np.ones((70, K), np.float32)
    X[35:] = -1.0
    X[69, ::2] = -1.0                                # mixed signs in one token
    w4 = []
    for j in range(130):
        if j % 3 == 0:
            w4.append(encode_q4K(0.5, 0.25, [63] * 8, [63] * 8, [15] * 256))
        elif j % 3 == 1:
            w4.append(encode_q4K(0.5, 0.0, [63] * 8, [0] * 8, [15 if e % 2 else 0 for e in range(256)]))
        else:
            w4.append(encode_q4K(0.5, 0.25, [0] * 8, [63] * 8, [0] * 256))
    W4 = np.stack([np.concatenate([b] * (K // 256)) for b in w4])
    w6 = []
    for j in range(130):
        if j % 2 == 0:
            w6.append(encode_q6K(0.5, [-128] * 16, [-32] * 256))
        else:
            w6.append(encode_q6K(0.5, [127] * 16, [31] * 256))
    W6 = np.stack([np.concatenate([b] * (K // 256)) for b in w6])
    xq, (q, _, _) = gpu_quantize(X)
    for wtype, W in (("q4_K", W4), ("q6_K", W6)):
        M, N = X.shape[0], W.shape[0]
        s = gpu_isums(wtype, W, xq, M, N, K)
        ref = O.isums(wtype, W, q)
        assert int(np.max(np.abs(ref))) == (15 * 127 * 32 if wtype == "q4_K" else 32 * 127 * 16)
        assert np.array_equal(s, ref), wtype
        check_out(gpu_mmq(wtype, W, X, N), O.mmq(wtype, W, X), f"extreme {wtype}")
    wp = B.q6K_prepare(dev(W6.reshape(-1)), 130, K)
    y = B.mmq_q6K_prep_q8(wp, xq, 70, 130, K)
    torch.cuda.synchronize()
    check_out(y.cpu().numpy(), O.mmq("q6_K", W6, X), "extreme q6_K prepared")
    # expanded: a = sc * (q6 - 32) reaches -4064 and 4096, the ends of its digit range
    we = B.q6K_expand(dev(W6.reshape(-1)), 130, K)
    s = B.mmq_q6K_exp_csums(we, xq, 70, 130, K)
    y = B.mmq_q6K_exp_q8(we, xq, 70, 130, K)
    torch.cuda.synchronize()
    ref = O.q6K_chunk_sums(W6, q)
    assert int(np.max(np.abs(ref))) == 32 * 127 * 128 * 32
    assert np.array_equal(s.cpu().numpy(), ref)
    check_out(y.cpu().numpy(), O.mmq("q6_K", W6, X), "extreme q6_K expanded")
