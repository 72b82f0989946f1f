"""Hardware facts the MMQ kernels rest on, checked on the device through libqpg_calib.so.

* Operand and result layouts of the three matrix instructions the kernels use
  (v_mfma_i32_32x32x32_i8, v_mfma_i32_32x32x16_i8, v_mfma_f32_32x32x16_bf16): lane l holds
  row (A) / column (B) l & 31 and the K-group l >> 5; result register r of lane l is row
  8 (r >> 2) + 4 (l >> 5) + (r & 3), column l & 31. Each probe packs random matrices by that
  rule, runs one instruction on one wave, unpacks the result by the same rule and compares it
  with the plain product A B^T + C computed on the host: any other layout fails.
* The accumulator trick of the fold: an int32 product accumulated onto the bits of 1.5 * 2^23
  reads as the f32 value 1.5 * 2^23 + I exactly, at the largest |I| each weight format
  reaches (15 * 127 * 32 for q4_K, 32 * 127 * 16 for q6_K).
* LDS-direct loads (buffer_load_dword[x4] with the LDS flag), which stage every tile: lane L's
  4 / 16 bytes land at LDS byte 4 L / 16 L, each lane's own source offset is honoured --
  permutations, and offsets that are not multiples of 4 (the raw q6_K staging reads rows that
  start 2 bytes past a 4-byte boundary) -- and bytes past the descriptor's range read as zero
  (rows and tokens past the matrix).
* v_permlane32_swap (the raw q6_K kernel's exchange of operand pieces between lane halves):
  register a's lanes 32..63 trade places with register b's lanes 0..31.
"""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALIB = os.path.join(ROOT, "quantized_prefill_gemm_amd", "libqpg_calib.so")
DEV = torch.device("cuda:0")
MAGIC_BITS = 0x4B400000


@pytest.fixture(scope="module")
def probe():
    lib = ctypes.CDLL(CALIB)
    f = lib.qpg_probe_mfma
    f.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5
    f.restype = ctypes.c_int

    def run(kind, a_lanes, b_lanes, c_lanes):
        a = torch.from_numpy(np.ascontiguousarray(a_lanes)).to(DEV)
        b = torch.from_numpy(np.ascontiguousarray(b_lanes)).to(DEV)
        c = torch.from_numpy(np.ascontiguousarray(c_lanes)).to(DEV)
        d = torch.empty_like(c)
        rc = f(kind, a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), None)
        assert rc == 0
        torch.cuda.synchronize()
        return d.cpu().numpy()
    return run


def pack_ab(mat, kgroup):
    """[32][K] matrix -> lane-major operand: lane l = row l & 31, k in kgroup*(l >> 5) + [0, kgroup)."""
    lanes = np.empty((64, kgroup), mat.dtype)
    for l in range(64):
        lanes[l] = mat[l & 31, kgroup * (l >> 5): kgroup * (l >> 5) + kgroup]
    return lanes


def c_row(r, l):
    return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)


def pack_c(mat):
    lanes = np.empty((64, 16), mat.dtype)
    for l in range(64):
        for r in range(16):
            lanes[l, r] = mat[c_row(r, l), l & 31]
    return lanes


def unpack_c(lanes):
    mat = np.empty((32, 32), lanes.dtype)
    for l in range(64):
        for r in range(16):
            mat[c_row(r, l), l & 31] = lanes[l, r]
    return mat


@pytest.mark.parametrize("kind,K", [(0, 32), (1, 16)])
def test_int8_layouts(probe, kind, K):
    rng = np.random.default_rng(100 + kind)
    A = rng.integers(-128, 128, size=(32, K)).astype(np.int8)
    B = rng.integers(-128, 128, size=(32, K)).astype(np.int8)
    C = rng.integers(-2 ** 20, 2 ** 20, size=(32, 32)).astype(np.int32)
    kg = K // 2
    d = probe(kind, pack_ab(A, kg), pack_ab(B, kg), pack_c(C))
    ref = A.astype(np.int64) @ B.astype(np.int64).T + C
    assert np.array_equal(unpack_c(d).astype(np.int64), ref)


def test_bf16_layout(probe):
    rng = np.random.default_rng(102)
    # small integers: every product and partial sum is exact in f32, so the result is unique
    A = rng.integers(-64, 64, size=(32, 16)).astype(np.float32)
    B = rng.integers(-64, 64, size=(32, 16)).astype(np.float32)
    C = rng.integers(-4096, 4096, size=(32, 32)).astype(np.float32)
    bf = lambda m: (m.view(np.uint32) >> 16).astype(np.uint16)     # exact: integers below 2^8
    d = probe(2, pack_ab(bf(A), 8), pack_ab(bf(B), 8), pack_c(C))
    ref = A.astype(np.float64) @ B.astype(np.float64).T + C
    assert np.array_equal(unpack_c(d).astype(np.float64), ref)


@pytest.mark.parametrize("kind,K,wmax,wmin", [(0, 32, 15, 0), (1, 16, 31, -32)])
def test_magic_accumulator_exact_at_extremes(probe, kind, K, wmax, wmin):
    """Weights at the ends of their range against activations of +-127 (and a mixed row):
    every int32 sum, written onto the bits of 1.5 * 2^23, reads as 1.5 * 2^23 + I exactly."""
    W = np.empty((32, K), np.int8)
    W[:16] = wmax
    W[16:] = wmin
    X = np.empty((32, K), np.int8)
    X[:11] = 127
    X[11:22] = -127
    X[22:] = np.where(np.arange(K) % 2 == 0, 127, -127)
    kg = K // 2
    C = np.full((32, 32), MAGIC_BITS, np.int32)
    d = unpack_c(probe(kind, pack_ab(W, kg), pack_ab(X, kg), pack_c(C)))
    I = W.astype(np.int64) @ X.astype(np.int64).T
    assert np.max(np.abs(I)) == (15 * 127 * 32 if kind == 0 else 32 * 127 * 16)
    as_f32 = d.view(np.float32).astype(np.float64)
    assert np.array_equal(as_f32, 1.5 * 2.0 ** 23 + I)
    assert np.array_equal(d.astype(np.int64) - MAGIC_BITS, I)


def test_step_probe_runs():
    """The compute-step probe (all modes, 1-4 waves per SIMD) reports a tick count for every
    workgroup."""
    lib = ctypes.CDLL(CALIB)
    lib.qpg_calib_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.qpg_calib_step.restype = ctypes.c_int
    lib.qpg_calib_step_blocks.argtypes = [ctypes.c_int]
    lib.qpg_calib_step_blocks.restype = ctypes.c_int64
    for w in (1, 2, 3, 4):
        nb = lib.qpg_calib_step_blocks(w)
        assert nb == torch.cuda.get_device_properties(0).multi_processor_count * w
        out = torch.zeros(nb * 4, dtype=torch.int64, device=DEV)
        for mode in range(8):
            assert lib.qpg_calib_step(mode, w, 20, ctypes.c_void_p(out.data_ptr()), None) == 0
            torch.cuda.synchronize()
            v = out.view(nb, 4).cpu().numpy()
            assert (v[:, 0] > 0).all() and (v[:, 1] > 0).all() and (v[:, 3] == 0).all()


def test_lds_direct_loads():
    lib = ctypes.CDLL(CALIB)
    f = lib.qpg_probe_lds_dma
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    src_np = ((np.arange(2048) * 7 + 3) & 255).astype(np.uint8)
    src = torch.from_numpy(src_np).to(DEV)

    def run(width, voff, nbytes):
        v = torch.tensor(voff, dtype=torch.int32, device=DEV)
        out = torch.zeros(256, dtype=torch.int32, device=DEV)
        assert f(width, src.data_ptr(), nbytes, v.data_ptr(), out.data_ptr(), None) == 0
        torch.cuda.synchronize()
        return out.cpu().numpy().view(np.uint8)

    def expect(width, voff, nbytes):
        e = np.frombuffer(np.full(256, 0xDEADBEEF, np.uint32).tobytes(), np.uint8).copy()
        for lane, o in enumerate(voff):
            for b in range(width):
                e[width * lane + b] = src_np[o + b] if o + b < nbytes else 0
        return e

    cases = [(4, [4 * l for l in range(64)], 2048),                    # identity
             (4, [4 * ((l * 37) % 64) for l in range(64)], 2048),      # a permutation of dwords
             (16, [16 * ((l * 29) % 64) for l in range(64)], 2048),    # a permutation of granules
             (4, [4 * l + 2 for l in range(64)], 2048),                # 2 bytes past 4-byte boundaries
             (4, [4 * l + 1 for l in range(64)], 2048),
             (16, [16 * l + 2 for l in range(64)], 2048),
             (16, [16 * l + 6 for l in range(64)], 2048),
             (16, [16 * l for l in range(64)], 100),                   # past the range: zeros
             # raw q6_K rows: 8 rows of 210-byte blocks, 8 dwords each from byte 2 of the row
             (4, [(l >> 3) * 210 + 2 + 4 * (l & 7) for l in range(64)], 2048)]
    for width, voff, nbytes in cases:
        got = run(width, voff, nbytes)
        assert np.array_equal(got, expect(width, voff, nbytes)), (width, voff[:3], nbytes)


def test_permlane32_swap():
    lib = ctypes.CDLL(CALIB)
    f = lib.qpg_probe_permlane32_swap
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    a = np.arange(64, dtype=np.uint32) * 7 + 1000
    b = np.arange(64, dtype=np.uint32) * 13 + 5000
    inp = torch.from_numpy(np.concatenate([a, b]).view(np.int32)).to(DEV)
    out = torch.zeros(128, dtype=torch.int32, device=DEV)
    assert f(inp.data_ptr(), out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(o[:64], np.concatenate([a[:32], b[:32]]))
    assert np.array_equal(o[64:], np.concatenate([a[32:], b[32:]]))
