"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the passage it follows. The pages print no worked example, so the
pins are closed forms derived by hand (tests/golden), layout sweeps against the
independently written encoders of tests/qblocks.py, a library routine for the fp16
rounding, exact rational arithmetic for the q8_1 rounding, brute force over the plain
definition Y = dequant(W) . dequant(q8_1(X))^T, and exact invariants.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from qblocks import encode_q4K, encode_q6K, f16_bits, near_tie_blocks
from quantized_prefill_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DA1 = 1032 * 2.0 ** -17          # fp16(1/127), derived in golden/closed_forms.json
DA127 = DA1 * 127                # 0.99993896484375


# ----------------------------------------------------------------------------- fp16

def test_f16_decode_all_patterns():
    """Every finite binary16 pattern decodes to numpy's value (library routine)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isinf(got[np.isinf(ref)]))


def test_f16_encode_matches_numpy_rne():
    """f32 -> fp16 round-to-nearest-even equals numpy's cast, incl. ties and subnormals."""
    rng = np.random.default_rng(7)
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
            2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 / 127, 31 / 127]
    vals += list(rng.uniform(-70000, 70000, 3000)) + list(rng.standard_normal(3000) * 1e-4)
    vals += list(np.exp(rng.uniform(-20, 11, 3000)))
    # exact ties between adjacent fp16 values
    h = rng.integers(0, 0x7bff, 2000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    vals += list((lo + hi) / 2)
    x = np.array(vals, np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------- q8_1

def test_q8_1_ties_golden():
    """amax = 127 gives d = 1: q = round half away from zero (golden/q8_1_ties.json)."""
    g = json.load(open(os.path.join(GOLDEN, "q8_1_ties.json")))
    x = np.array([g["x"]], np.float32)
    q, dh, ss = O.quantize_q8_1(x)
    assert q[0].tolist() == g["q"]
    assert int(ss[0, 0]) == g["ssum"]
    assert int(dh[0, 0]) == g["dh_bits"]


def test_q8_1_zero_block():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    q, dh, ss = O.quantize_q8_1(x)
    assert not q[0].any() and not q[1, :32].any()
    assert dh[0].tolist() == [0, 0] and ss[0].tolist() == [0, 0] and dh[1, 0] == 0 and ss[1, 0] == 0
    assert q[1, 32] == -127 and q[1, 63] == 127


def test_q8_1_ramp_exact_rationals():
    """x = s*k for k = 0..31: q = round(k*127/31) computed with exact fractions.

    The f32 path (d = amax/127, 1/d, x*(1/d)) stays within a few ulp of the exact ratio,
    and every exact ratio here is at least 1e-3 away from a rounding tie, so the f32
    result must equal the exact rounding. Scaling by powers of two must not change q."""
    for scale in (1.0, 2.0 ** -6, 2.0 ** 9):
        x = (np.arange(32, dtype=np.float32) * np.float32(scale))[None, :]
        q, dh, ss = O.quantize_q8_1(x)
        exp = []
        for k in range(32):
            r = Fraction(k * 127, 31)
            fl = r.numerator // r.denominator
            frac = r - fl
            assert abs(frac - Fraction(1, 2)) > Fraction(1, 1000)
            exp.append(fl + (1 if frac > Fraction(1, 2) else 0))
        assert q[0].tolist() == exp
        assert int(ss[0, 0]) == sum(exp)
        d = np.float32(np.float32(31 * scale) / np.float32(127))   # IEEE f32 division (numpy)
        assert int(dh[0, 0]) == int(np.array(d, np.float16).view(np.uint16))


@pytest.mark.parametrize("amax", [127.0, 63.5, 127.0 * 2.0 ** -20])
def test_q8_1_near_ties_exact(amax):
    """Blocks whose scale d = amax/127 is a power of two, so x * (1/d) is exact and q must be
    the exact rational x/d rounded half away from zero: values at n + 1/2 and up to three f32
    steps either side, n = 0..126, both signs (the quantiser's rounding reading)."""
    x = near_tie_blocks(amax)
    q, dh, ss = O.quantize_q8_1(x)
    d = Fraction(amax) / 127
    flat = x.reshape(-1)
    exp = np.empty(flat.size, np.int64)
    for i, v in enumerate(flat.tolist()):
        r = abs(Fraction(v) / d)
        n = r.numerator // r.denominator
        n += 1 if r - n >= Fraction(1, 2) else 0
        exp[i] = n if v >= 0 else -n
    assert np.array_equal(q.reshape(-1).astype(np.int64), exp)
    blocks = exp.reshape(-1, 32)
    assert np.array_equal(ss.reshape(-1).astype(np.int64), blocks.sum(axis=1))
    assert np.count_nonzero(np.abs(blocks[:, 1:]) >= 1) > 1500


def test_q8_1_negation_and_bounds():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 256)).astype(np.float32) * 3
    q, dh, ss = O.quantize_q8_1(x)
    qn, dhn, ssn = O.quantize_q8_1(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dhn, dh) and np.array_equal(ssn, -ss)
    assert q.max() == 127 or q.min() == -127
    assert np.abs(q.astype(int)).max() <= 127
    # each block's largest |x| maps to +-127
    blocks = np.abs(q.reshape(5, 8, 32)).max(axis=2)
    assert np.all(blocks == 127)
    assert np.array_equal(ss, q.reshape(5, 8, 32).astype(np.int32).sum(axis=2))


# ----------------------------------------------------------------------------- decoders

def test_q4K_decoder_roundtrip_random_fields():
    """Random field values, encoded by the bit table of qblocks, decode unchanged."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        nib = rng.integers(0, 16, 256)
        d, dmin = float(np.float16(rng.uniform(1e-3, 1))), float(np.float16(rng.uniform(0, 1)))
        blk = encode_q4K(d, dmin, sc, m, nib)
        dd, ddm, sc2, m2, nib2 = O.decode_q4K(blk)
        assert dd == d and ddm == dmin
        assert sc2.tolist() == sc.tolist() and m2.tolist() == m.tolist()
        assert nib2.tolist() == nib.tolist()


def test_q6K_decoder_roundtrip_random_fields():
    rng = np.random.default_rng(12)
    for _ in range(200):
        sc = rng.integers(-128, 128, 16)
        v = rng.integers(-32, 32, 256)
        d = float(np.float16(rng.uniform(1e-3, 1)))
        blk = encode_q6K(d, sc, v)
        dd, sc2, v2 = O.decode_q6K(blk)
        assert dd == d and sc2.tolist() == sc.tolist() and v2.tolist() == v.tolist()


def test_q4K_nibble_placement_from_pages():
    """qs byte 32*p + l holds element l of sub-block 2p (low nibble) and of 2p+1 (high
    nibble) -- the B-unpack rule p = sg>>1, is_hi = sg&1 (page 'r29 - NB kd-loop unroll',
    sec. 3.2). Checked directly on raw bytes, without the test encoder."""
    blk = np.zeros(144, np.uint8)
    blk[16:144] = np.arange(128, dtype=np.uint8) * 37 + 5
    _, _, _, _, nib = O.decode_q4K(blk)
    qs = blk[16:144].astype(int)
    for s in range(8):
        p, hi = s >> 1, s & 1
        for l in range(32):
            byte = qs[32 * p + l]
            assert nib[32 * s + l] == ((byte >> 4) & 15 if hi else byte & 15)


# ----------------------------------------------------------------------------- closed forms

def _const_q4K_row(K, d, dmin, sc, m, nib):
    blk = encode_q4K(d, dmin, [sc] * 8, [m] * 8, [nib] * 256)
    return np.tile(blk, K // 256)[None, :]


def _const_q6K_row(K, d, sc, v):
    blk = encode_q6K(d, [sc] * 16, [v] * 256)
    return np.tile(blk, K // 256)[None, :]


def test_closed_forms_golden():
    g = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))
    for case in g["cases"]:
        K = case["K"]
        if case["wtype"] == "q4_K":
            w = _const_q4K_row(K, case["d"], case["dmin"], case["sc"], case["m"], case["nib"])
        else:
            w = _const_q6K_row(K, case["d"], case["sc"], case["v"])
        x = np.ones((3, K), np.float32)
        y = O.mmq(case["wtype"], w, x, nthreads=1)
        assert np.all(y == case["expected"]), (case["name"], y)
        yb = O.brute_force(case["wtype"], w, x)
        assert np.allclose(yb, case["expected"], rtol=1e-14, atol=0), case["name"]


# ----------------------------------------------------------------------------- layout sweeps

def test_q4K_one_hot_recovers_nibbles():
    """Token i one-hot at k = i: Y[i, j] = (d*sc*nib[j,i] - dmin*m) * fp16(1/127) * 127."""
    rng = np.random.default_rng(21)
    N, K = 8, 256
    nibs = rng.integers(0, 16, (N, K))
    w = np.stack([encode_q4K(1.0, 0.0, [1] * 8, [0] * 8, nibs[j]) for j in range(N)])
    x = np.eye(K, dtype=np.float32)
    y = O.mmq("q4_K", w, x, nthreads=2)
    assert np.array_equal(y, DA127 * nibs.T.astype(np.float64))


def test_q4K_scale_min_sweep():
    """nib = 1 everywhere, distinct (sc_s, m_s) >= 16 per sub-block (so the top two bits
    of every field are exercised), one-hot token per sub-block:
    Y[s, 0] = (d*sc_s - dmin*m_s) * fp16(2/127) * 127, with fp16(2/127) = 2 * fp16(1/127)."""
    sc = [17, 63, 40, 33, 48, 21, 59, 30]
    m = [50, 16, 61, 26, 35, 63, 19, 44]
    d, dmin = 0.25, 0.125
    w = encode_q4K(d, dmin, sc, m, [1] * 256)[None, :]
    x = np.zeros((8, 256), np.float32)
    for s in range(8):
        x[s, 32 * s + 3] = 2.0
    y = O.mmq("q4_K", w, x, nthreads=1)
    for s in range(8):
        assert y[s, 0] == (d * sc[s] - dmin * m[s]) * 2 * DA127


def test_q6K_one_hot_recovers_values():
    rng = np.random.default_rng(22)
    N, K = 6, 256
    v = rng.integers(-32, 32, (N, K))
    w = np.stack([encode_q6K(1.0, [1] * 16, v[j]) for j in range(N)])
    y = O.mmq("q6_K", w, np.eye(K, dtype=np.float32), nthreads=2)
    assert np.array_equal(y, DA127 * v.T.astype(np.float64))


def test_q6K_signed_scale_sweep():
    sc = [-64, 63, -1, 1, 17, -33, 5, -7, 127, -128, 2, -2, 40, -40, 9, -9]
    w = encode_q6K(0.5, sc, [31] * 256)[None, :]
    x = np.zeros((16, 256), np.float32)
    for u in range(16):
        x[u, 16 * u + 5] = 1.0
    y = O.mmq("q6_K", w, x, nthreads=1)
    for u in range(16):
        assert y[u, 0] == 0.5 * sc[u] * 31 * DA127


def test_q6K_chunk_sums_one_hot_and_closed_form():
    """Scale-weighted chunk sums from encoder-chosen fields: a one-hot activation at k gives
    sc[k/16] * v[k] * 127 in chunk k/32 and zero elsewhere; constant blocks give the closed
    form 32 * 127 * sc * v; and the chunk sums fold to the oracle's output."""
    rng = np.random.default_rng(23)
    N, K = 5, 512
    sc = rng.integers(-128, 128, (N, K // 16))
    v = rng.integers(-32, 32, (N, K))
    w = np.stack([np.concatenate([encode_q6K(0.25, sc[j, 16 * b:16 * b + 16], v[j, 256 * b:256 * b + 256])
                                  for b in range(K // 256)]) for j in range(N)])
    q, _, _ = O.quantize_q8_1(np.eye(K, dtype=np.float32))      # q = 127 on the diagonal
    C = O.q6K_chunk_sums(w, q, nthreads=2)
    assert C.shape == (K, N, K // 32)
    for k in range(K):
        want = np.zeros((N, K // 32), np.int64)
        want[:, k // 32] = sc[:, k // 16] * v[:, k] * 127
        assert np.array_equal(C[k], want), k
    wc = np.stack([np.concatenate([encode_q6K(1.0, [-128] * 16, [-32] * 256)] * 2),
                   np.concatenate([encode_q6K(1.0, [127] * 16, [31] * 256)] * 2)])
    qc, dh, ss = O.quantize_q8_1(np.ones((3, K), np.float32))
    Cc = O.q6K_chunk_sums(wc, qc, nthreads=1)
    assert np.all(Cc[:, 0] == 32 * 127 * 128 * 32) and np.all(Cc[:, 1] == 32 * 127 * 127 * 31)
    # folding the chunk sums with da and d reproduces the oracle's q6_K output
    W, X = inputs.small_case("q6_K", 9, 7, 768, seed=4, gain=True)
    q, dh, ss = O.quantize_q8_1(X)
    C = O.q6K_chunk_sums(W, q, nthreads=2).astype(np.float64)
    da = np.vectorize(O.f16_to_f64, otypes=[np.float64])(dh)                    # [M, K/32]
    d = np.array([[O.decode_q6K(W[j, 210 * b:210 * b + 210])[0] for b in range(768 // 256)]
                  for j in range(7)])                                           # [N, K/256]
    y = np.einsum("ic,jc,ijc->ij", da, np.repeat(d, 8, axis=1), C)
    r = O.mmq("q6_K", W, X, nthreads=2)
    assert np.allclose(y, r, rtol=1e-12, atol=1e-9 * np.abs(r).max())


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (7, 5, 256), (33, 17, 512), (64, 40, 768)])
def test_factored_equals_brute_force(wtype, M, N, K):
    """Exact integer sums + fold == dequant(W) . dequant(q8_1(X))^T (fp64) to 1e-12."""
    W, X = inputs.small_case(wtype, M, N, K, seed=1, gain=True)
    y = O.mmq(wtype, W, X, nthreads=4)
    yb = O.brute_force(wtype, W, X)
    scale = np.max(np.abs(yb))
    assert np.max(np.abs(y - yb)) <= 1e-12 * scale


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
def test_isums_against_known_construction(wtype):
    """Integer sums from the encoder's own values (numpy integer products)."""
    rng = np.random.default_rng(31)
    M, N, K = 5, 4, 512
    if wtype == "q4_K":
        vals = rng.integers(0, 16, (N, K))
        w = np.stack([np.concatenate([encode_q4K(0.5, 0.25, rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                                                 vals[j, b * 256:(b + 1) * 256]) for b in range(K // 256)])
                      for j in range(N)])
        per = 32
    else:
        vals = rng.integers(-32, 32, (N, K))
        w = np.stack([np.concatenate([encode_q6K(0.5, rng.integers(-64, 64, 16), vals[j, b * 256:(b + 1) * 256])
                                      for b in range(K // 256)]) for j in range(N)])
        per = 16
    q = rng.integers(-127, 128, (M, K)).astype(np.int8)
    s = O.isums(wtype, w, q, nthreads=2)
    ref = np.einsum("ick,jck->ijc", q.astype(np.int64).reshape(M, K // per, per),
                    vals.astype(np.int64).reshape(N, K // per, per))
    assert np.array_equal(s, ref)


# ----------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
def test_invariants(wtype):
    W, X = inputs.small_case(wtype, 16, 12, 512, seed=2)
    y = O.mmq(wtype, W, X)
    assert np.array_equal(O.mmq(wtype, W, -X), -y)                  # Y(-X) = -Y(X)
    for t in (-3, 5):
        assert np.array_equal(O.mmq(wtype, W, X * np.float32(2.0 ** t)), y * 2.0 ** t)
    # isums of K = 512 are the concatenation of the two K = 256 halves
    q, _, _ = O.quantize_q8_1(X)
    bs = 144 if wtype == "q4_K" else 210
    s = O.isums(wtype, W, q)
    s0 = O.isums(wtype, W[:, :bs], q[:, :256])
    s1 = O.isums(wtype, W[:, bs:], q[:, 256:])
    assert np.array_equal(s, np.concatenate([s0, s1], axis=2))


def test_weight_scale_power_of_two():
    """Scaling every q4_K d and dmin by 2^t scales Y by 2^t exactly."""
    rng = np.random.default_rng(5)
    sc = rng.integers(0, 64, (3, 8))
    m = rng.integers(0, 64, (3, 8))
    nib = rng.integers(0, 16, (3, 256))
    X = rng.standard_normal((9, 256)).astype(np.float32)
    w1 = np.stack([encode_q4K(0.00390625 * 3, 0.0078125 * 5, sc[j], m[j], nib[j]) for j in range(3)])
    w2 = np.stack([encode_q4K(0.00390625 * 3 * 8, 0.0078125 * 5 * 8, sc[j], m[j], nib[j]) for j in range(3)])
    assert np.array_equal(O.mmq("q4_K", w2, X), 8 * O.mmq("q4_K", w1, X))


def test_oracle_detects_planted_mistakes():
    """A plausible mistake in the fold shows at the 1e0 scale, far above the 1e-3 bar.
    (Planted on the CPU in a copy of the fold written here, not in the GPU path.)"""
    W, X = inputs.small_case("q4_K", 8, 8, 256, seed=4)
    q, dh, ss = O.quantize_q8_1(X)
    y = O.mmq_q8("q4_K", W, q, dh, ss)
    yb = O.brute_force("q4_K", W, X)
    s = np.sqrt(np.mean(yb ** 2))
    assert np.max(np.abs(y - yb)) < 1e-10 * s
    # dropping the min term, or using the unsigned nibble without the min, is a 1e0 error
    s_int = O.isums("q4_K", W, q)
    da = np.vectorize(O.f16_to_f64)(dh)
    dsv = np.zeros((8, 8))
    for j in range(8):
        d, dmin, sc, m, _ = O.decode_q4K(W[j])
        dsv[j] = d * sc
    no_min = np.einsum("ic,jc,ijc->ij", da, dsv, s_int)
    assert np.max(np.abs(no_min - yb)) > 0.1 * s


def test_q8_1_overflowing_inverse_scale():
    """A block of f32 subnormals: d = amax/127 < 2^-128, so 1/d = inf; x*(1/d) saturates to
    +-127 and x = 0 stays 0; fp16(d) = 0 so the block contributes nothing downstream."""
    x = np.zeros((1, 32), np.float32)
    x[0, :16] = np.float32(3e-40) * np.arange(1, 17, dtype=np.float32)
    x[0, 16:31] = -np.float32(2e-40) * np.arange(1, 16, dtype=np.float32)
    q, dh, ss = O.quantize_q8_1(x)
    assert q[0, :16].tolist() == [127] * 16
    assert q[0, 16:31].tolist() == [-127] * 15
    assert q[0, 31] == 0
    assert dh[0, 0] == 0 and ss[0, 0] == 127 * 16 - 127 * 15
