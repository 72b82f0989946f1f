"""Host-side checks of the C ABI (no kernel is ever launched here).

The library must load, export every function include/qpg.h declares, and reject bad
arguments with the documented status before touching the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qpg.h")
LIB = os.path.join(ROOT, "quantized_prefill_gemm_amd", "libqpg.so")

EINVAL, EALIGN, EDEVICE = -1, -2, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9A-Z]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.skip("libqpg.so not built")
    lib = ctypes.CDLL(LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.qpg_strerror.restype = ctypes.c_char_p
    lib.qpg_q8_1_bytes.restype = ctypes.c_size_t
    lib.qpg_q8_1_bytes.argtypes = [I64, I64]
    lib.quantize_q8_1.argtypes = [P, P, I64, I64, P]
    for f in (lib.mmq_q4K, lib.mmq_q6K):
        f.argtypes = [P, P, P, I64, I64, I64, P, P]
    for f in (lib.mmq_q4K_q8, lib.mmq_q6K_q8, lib.mmq_q4K_isums, lib.mmq_q6K_isums, lib.mmq_q6K_prep_q8,
              lib.mmq_q6K_prep_isums):
        f.argtypes = [P, P, P, I64, I64, I64, P]
    lib.qpg_q6K_prep_bytes.restype = ctypes.c_size_t
    lib.qpg_q6K_prep_bytes.argtypes = [I64, I64]
    lib.q6K_prepare.argtypes = [P, P, I64, I64, P]
    lib.qpg_q6K_exp_bytes.restype = ctypes.c_size_t
    lib.qpg_q6K_exp_bytes.argtypes = [I64, I64]
    lib.q6K_expand.argtypes = [P, P, I64, I64, P]
    for f in (lib.mmq_q6K_exp_q8, lib.mmq_q6K_exp_csums):
        f.argtypes = [P, P, P, I64, I64, I64, P]
    lib.qpg_mmq_sk_bytes.restype = ctypes.c_size_t
    lib.qpg_mmq_sk_bytes.argtypes = [I64, I64, I64, ctypes.c_int]
    for f in (lib.mmq_q4K_q8_sk, lib.mmq_q6K_q8_sk, lib.mmq_q6K_prep_q8_sk, lib.mmq_q6K_exp_q8_sk):
        f.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.mmq_q4K_noalloc.argtypes = [P, P, P, I64, I64, I64, P]
    lib.mmq_q4K_noalloc.restype = ctypes.c_int
    return lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("quantize_q8_1", "mmq_q4K", "mmq_q6K", "mmq_q4K_q8", "mmq_q6K_q8", "mmq_q4K_isums",
              "mmq_q6K_isums", "qpg_q8_1_bytes", "qpg_strerror"):
        assert n in names, n


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_binding_names_match_header():
    from quantized_prefill_gemm_amd import binding
    assert set(declared_functions()) == set(binding.EXPORTS)


def test_strerror_and_sizes(L):
    for code in (0, -1, -2, -3, -4, -99):
        assert L.qpg_strerror(code)
    assert L.qpg_q8_1_bytes(512, 4096) == 512 * 4096 + 4 * 512 * 128
    assert L.qpg_q8_1_bytes(1, 32) == 36
    assert L.qpg_q8_1_bytes(0, 256) == 0
    assert L.qpg_q8_1_bytes(4, 48) == 0


A16 = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced: every call below fails validation
A1 = ctypes.c_void_p((1 << 20) + 1)
A2 = ctypes.c_void_p((1 << 20) + 2)
A8 = ctypes.c_void_p((1 << 20) + 8)


@pytest.mark.parametrize("args,expect", [
    ((None, A16, 4, 256), EINVAL),
    ((A16, None, 4, 256), EINVAL),
    ((A16, A16, 0, 256), EINVAL),
    ((A16, A16, 4, 0), EINVAL),
    ((A16, A16, 4, 48), EINVAL),
    ((A16, A16, 1 << 31, 256), EINVAL),
    ((A8, A16, 4, 256), EALIGN),
    ((A16, A8, 4, 256), EALIGN),
])
def test_quantize_rejects(L, args, expect):
    assert L.quantize_q8_1(*args, None) == expect


@pytest.mark.parametrize("fn", ["mmq_q4K_q8", "mmq_q6K_q8", "mmq_q4K_isums", "mmq_q6K_isums", "mmq_q6K_prep_q8",
                                "mmq_q6K_prep_isums", "mmq_q6K_exp_q8", "mmq_q6K_exp_csums"])
@pytest.mark.parametrize("args,expect", [
    ((None, A16, A16, 64, 256, 256), EINVAL),
    ((A16, None, A16, 64, 256, 256), EINVAL),
    ((A16, A16, None, 64, 256, 256), EINVAL),
    ((A16, A16, A16, 0, 256, 256), EINVAL),
    ((A16, A16, A16, 64, 0, 256), EINVAL),
    ((A16, A16, A16, 64, 256, 128), EINVAL),
    ((A16, A16, A16, 64, 256, 288), EINVAL),
    ((A16, A16, A16, 64, 1 << 31, 256), EINVAL),
    ((A16, A8, A16, 64, 256, 256), EALIGN),
])
def test_mmq_q8_rejects(L, fn, args, expect):
    assert getattr(L, fn)(*args, None) == expect


def test_alignment_rules_per_type(L):
    # q4_K weights need 16-byte alignment, raw q6_K weights 2-byte (the block's fp16 d)
    assert L.mmq_q4K_q8(A8, A16, A16, 64, 256, 256, None) == EALIGN
    assert L.mmq_q6K_q8(A1, A16, A16, 64, 256, 256, None) == EALIGN
    assert L.mmq_q6K_isums(A1, A16, A16, 64, 256, 256, None) == EALIGN
    assert L.mmq_q6K(A1, A16, A16, 64, 256, 256, A16, None) == EALIGN
    assert L.mmq_q4K(A16, A8, A16, 64, 256, 256, A16, None) == EALIGN     # x
    assert L.mmq_q4K(A16, A16, A16, 64, 256, 256, A8, None) == EALIGN     # workspace
    assert L.mmq_q6K(A16, A16, A16, 64, 256, 256, None, None) == EINVAL   # missing workspace


def test_q6K_prepare_sizes_and_rejects(L):
    # 32 KiB per (128-row tile, super-block)
    assert L.qpg_q6K_prep_bytes(4096, 11008) == 32 * 43 * 32768
    assert L.qpg_q6K_prep_bytes(129, 256) == 2 * 1 * 32768
    assert L.qpg_q6K_prep_bytes(1, 512) == 2 * 32768
    for n, k in ((0, 256), (128, 0), (128, 300), (128, 128), (1 << 31, 256), (128, 1 << 24)):
        assert L.qpg_q6K_prep_bytes(n, k) == 0
    assert L.q6K_prepare(None, A16, 128, 256, None) == EINVAL
    assert L.q6K_prepare(A16, None, 128, 256, None) == EINVAL
    assert L.q6K_prepare(A16, A16, 0, 256, None) == EINVAL
    assert L.q6K_prepare(A16, A16, 128, 288, None) == EINVAL
    assert L.q6K_prepare(A2, A16, 128, 256, None) == EALIGN     # raw blocks need 4-byte alignment
    assert L.q6K_prepare(A16, A8, 128, 256, None) == EALIGN     # prepared layout needs 16
    assert L.mmq_q6K_prep_q8(A8, A16, A16, 64, 256, 256, None) == EALIGN
    assert L.mmq_q6K_prep_q8(A16, A16, A16, 64, 256, 1 << 24, None) == EINVAL


def test_q6K_expand_sizes_and_rejects(L):
    # 35,072 bytes per (64-row tile, super-block): two 17 KiB digit images and d per row
    assert L.qpg_q6K_exp_bytes(4096, 11008) == 64 * 43 * 35072
    assert L.qpg_q6K_exp_bytes(65, 256) == 2 * 1 * 35072
    assert L.qpg_q6K_exp_bytes(1, 512) == 2 * 35072
    for n, k in ((0, 256), (64, 0), (64, 300), (64, 128), (1 << 31, 256), (64, 1 << 24)):
        assert L.qpg_q6K_exp_bytes(n, k) == 0
    assert L.q6K_expand(None, A16, 64, 256, None) == EINVAL
    assert L.q6K_expand(A16, None, 64, 256, None) == EINVAL
    assert L.q6K_expand(A16, A16, 0, 256, None) == EINVAL
    assert L.q6K_expand(A16, A16, 64, 288, None) == EINVAL
    assert L.q6K_expand(A16, A8, 64, 256, None) == EALIGN      # expanded layout needs 16
    assert L.mmq_q6K_exp_q8(A8, A16, A16, 64, 256, 256, None) == EALIGN
    assert L.mmq_q6K_exp_q8(A16, A16, A16, 64, 256, 1 << 24, None) == EINVAL
    assert L.mmq_q6K_exp_csums(A16, A16, A2, 64, 256, 256, None) == EALIGN


def test_splitk_workspace_sizes(L):
    # P = min(8, 256 // tiles, (K/256) // 3) when tiles <= 128, else no split (0 bytes); when M
    # fits one tile height, P = min(8, 512 // tiles, K/256) instead. q4_K tiles are 32 x 128
    # when the 64 x 128 grid has <= 128 tiles (or M <= 256 and > 256 tiles)
    assert L.qpg_mmq_sk_bytes(512, 512, 4096, 0) == 4 * 512 * 512 * 4      # 64 tiles of 32 rows -> 4
    assert L.qpg_mmq_sk_bytes(512, 1376, 4096, 0) == 0                     # 176 tiles of 32 rows
    assert L.qpg_mmq_sk_bytes(16, 4096, 4096, 0) == 8 * 16 * 4096 * 4      # one row of 32 tiles -> 8
    assert L.qpg_mmq_sk_bytes(32, 11008, 4096, 0) == 5 * 32 * 11008 * 4    # one row of 86 tiles -> 5
    assert L.qpg_mmq_sk_bytes(33, 4096, 4096, 0) == 4 * 33 * 4096 * 4      # two rows of 32 -> 4
    assert L.qpg_mmq_sk_bytes(64, 4096, 4096, 3) == 8 * 64 * 4096 * 4      # one row of 64 tiles (64 x 64) -> 8
    assert L.qpg_mmq_sk_bytes(16, 128, 512, 0) == 2 * 16 * 128 * 4         # one tile, 2 SB -> 2
    assert L.qpg_mmq_sk_bytes(16, 128, 256, 0) == 0                        # one super-block
    assert L.qpg_mmq_sk_bytes(512, 512, 4096, 1) == 5 * 512 * 512 * 4      # q6_K: 32 tiles of 64 rows -> 5
    assert L.qpg_mmq_sk_bytes(512, 512, 11008, 1) == 8 * 512 * 512 * 4     # 32 tiles, 43 SB -> 8
    assert L.qpg_mmq_sk_bytes(512, 512, 11008, 2) == 8 * 512 * 512 * 4
    assert L.qpg_mmq_sk_bytes(512, 512, 11008, 3) == 4 * 512 * 512 * 4     # 64 tiles of 64 x 64 -> 4
    assert L.qpg_mmq_sk_bytes(64, 100, 1536, 0) == 2 * 64 * 100 * 4        # 1 tile, 6 SB -> 2
    assert L.qpg_mmq_sk_bytes(512, 11008, 4096, 0) == 0                    # 688 tiles
    assert L.qpg_mmq_sk_bytes(512, 1024, 4096, 3) == 2 * 512 * 1024 * 4    # 128 tiles -> 256 / 128 = 2
    assert L.qpg_mmq_sk_bytes(512, 1088, 4096, 3) == 0                     # 136 tiles of 64 x 64
    assert L.qpg_mmq_sk_bytes(64, 128, 1280, 0) == 0                       # 5 SB: < 3 per piece
    for form in (-1, 4):
        assert L.qpg_mmq_sk_bytes(512, 512, 4096, form) == 0
    assert L.qpg_mmq_sk_bytes(512, 512, 300, 0) == 0
    assert L.qpg_mmq_sk_bytes(0, 512, 4096, 0) == 0


def test_splitk_rejects(L):
    need = L.qpg_mmq_sk_bytes(512, 512, 4096, 0)
    need6 = L.qpg_mmq_sk_bytes(512, 512, 4096, 1)
    assert need > 0 and need6 > 0
    assert L.mmq_q4K_q8_sk(A16, A16, A16, 512, 512, 4096, None, need, None) == EINVAL      # no workspace
    assert L.mmq_q4K_q8_sk(A16, A16, A16, 512, 512, 4096, A16, need - 4, None) == EINVAL  # too small
    assert L.mmq_q4K_q8_sk(A16, A16, A16, 512, 512, 4096, A8, need, None) == EALIGN
    assert L.mmq_q4K_q8_sk(A8, A16, A16, 512, 512, 4096, A16, need, None) == EALIGN
    assert L.mmq_q6K_q8_sk(A1, A16, A16, 512, 512, 4096, A16, need6, None) == EALIGN      # q6_K: 2 bytes
    assert L.mmq_q6K_prep_q8_sk(A16, A16, A16, 512, 512, 1 << 24, A16, need, None) == EINVAL
    assert L.mmq_q6K_exp_q8_sk(None, A16, A16, 512, 512, 4096, A16, need, None) == EINVAL
    assert L.mmq_q6K_exp_q8_sk(A16, A16, A16, 512, 512, 288, A16, need, None) == EINVAL


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="device check path is only exercised where no GPU exists")
def test_valid_call_without_device_reports_edevice(L):
    # All arguments valid: validation passes and the device query fails -> QPG_EDEVICE,
    # nothing is enqueued.
    assert L.mmq_q4K_q8(A16, A16, A16, 64, 256, 256, None) == EDEVICE
    assert L.quantize_q8_1(A16, A16, 64, 256, None) == EDEVICE
    assert L.q6K_prepare(A16, A16, 128, 256, None) == EDEVICE
    assert L.mmq_q6K_prep_q8(A16, A16, A16, 64, 256, 256, None) == EDEVICE
    assert L.q6K_expand(A2, A16, 64, 256, None) == EDEVICE          # raw blocks: any alignment
    assert L.mmq_q6K_q8(A2, A16, A16, 64, 256, 256, None) == EDEVICE  # raw q6_K MMQ: 2-byte blocks
    assert L.mmq_q6K(A2, A16, A16, 64, 256, 256, A16, None) == EDEVICE
    assert L.mmq_q6K_exp_q8(A16, A16, A16, 64, 256, 256, None) == EDEVICE
    # no split for this shape: the workspace may be absent
    assert L.mmq_q4K_q8_sk(A16, A16, A16, 64, 256, 1280, None, 0, None) == EDEVICE
    assert L.mmq_q6K_exp_q8_sk(A16, A16, A16, 64, 256, 4096, A16, 8 * 64 * 256 * 4, None) == EDEVICE


CALIB = os.path.join(ROOT, "quantized_prefill_gemm_amd", "libqpg_calib.so")
CALIB_HEADER = os.path.join(ROOT, "include", "qpg_calib.h")


def test_calib_library_exports_and_rejects():
    if not os.path.exists(CALIB):
        pytest.skip("libqpg_calib.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(CALIB_HEADER).read(), flags=re.S)
    names = re.findall(r"^\s*(?:int|int64_t)\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    assert names == ["qpg_calib_mfma_i8", "qpg_calib_step", "qpg_calib_step_blocks", "qpg_probe_mfma",
                     "qpg_probe_lds_dma", "qpg_probe_permlane32_swap"]
    lib = ctypes.CDLL(CALIB)
    for n in names:
        assert hasattr(lib, n), n
    st = lib.qpg_calib_step
    st.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    st.restype = ctypes.c_int
    assert st(8, 3, 100, A16, None) == EINVAL           # mode
    assert st(-1, 3, 100, A16, None) == EINVAL
    assert st(2, 0, 100, A16, None) == EINVAL           # waves per SIMD
    assert st(2, 5, 100, A16, None) == EINVAL
    assert st(2, 3, 0, A16, None) == EINVAL             # iters
    assert st(2, 3, 100, None, None) == EINVAL
    assert st(2, 3, 100, ctypes.c_void_p((1 << 20) + 4), None) == EALIGN
    pr = lib.qpg_probe_mfma
    pr.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5
    pr.restype = ctypes.c_int
    assert pr(3, A16, A16, A16, A16, None) == EINVAL
    assert pr(0, None, A16, A16, A16, None) == EINVAL
    assert pr(0, A8, A16, A16, A16, None) == EALIGN
    assert pr(2, A16, A16, A8, A16, None) == EALIGN
    dm = lib.qpg_probe_lds_dma
    dm.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    dm.restype = ctypes.c_int
    assert dm(8, A16, 1024, A16, A16, None) == EINVAL          # width
    assert dm(4, A16, 0, A16, A16, None) == EINVAL             # nbytes
    assert dm(4, None, 1024, A16, A16, None) == EINVAL
    assert dm(16, A8, 1024, A16, A16, None) == EALIGN          # src must be 16-byte aligned
    ps = lib.qpg_probe_permlane32_swap
    ps.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    ps.restype = ctypes.c_int
    assert ps(None, A16, None) == EINVAL
    assert ps(A16, ctypes.c_void_p((1 << 20) + 2), None) == EALIGN
    if not _has_gpu():
        assert ps(A16, A16, None) == EDEVICE
        assert dm(16, A16, 1024, A16, A16, None) == EDEVICE
        assert st(2, 3, 100, A16, None) == EDEVICE
        assert pr(1, A8, A8, A16, A16, None) == EDEVICE     # 8-byte operands suffice for kind 1
    f = lib.qpg_calib_mfma_i8
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(512, 100, None, None) == EINVAL
    assert f(0, 100, A16, None) == EINVAL
    assert f(65537, 100, A16, None) == EINVAL
    assert f(512, 0, A16, None) == EINVAL
    assert f(512, 10_000_001, A16, None) == EINVAL
    assert f(512, 100, ctypes.c_void_p((1 << 20) + 4), None) == EALIGN
    if not _has_gpu():
        assert f(512, 100, A16, None) == EDEVICE


# ---------------------------------------------------------------------------- binding checks
# The binding must refuse caller-supplied outputs that are too small (the C ABI takes no
# output size). Host-only: the is-a-device-tensor check and the stream lookup are bypassed,
# the size helpers come from the real library, and the compute entry points are replaced by
# a recorder, so a call that passes validation is seen without any kernel being launched.

@pytest.fixture
def recorded(monkeypatch, L):
    from quantized_prefill_gemm_amd import binding as Bd
    calls = []

    real = Bd.lib()

    class Recorder:
        def __getattr__(self, name):
            if name.startswith("qpg_"):
                return getattr(real, name)
            def f(*a):
                calls.append(name)
                return 0
            return f

    monkeypatch.setattr(Bd, "lib", lambda: Recorder())

    def dev_host(t, dtype, name):
        if t.dtype != dtype:
            raise Bd.QPGError(Bd.QPG_EINVAL, f"{name} dtype")
        if not t.is_contiguous():
            raise Bd.QPGError(Bd.QPG_EINVAL, f"{name} contiguity")

    monkeypatch.setattr(Bd, "_dev", dev_host)
    monkeypatch.setattr(Bd, "_stream", lambda stream=None: None)
    return Bd, calls


def test_binding_rejects_undersized_outputs(recorded):
    import torch
    Bd, calls = recorded
    M, N, K = 64, 200, 512
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    w4, w6 = u8(N * 2 * 144), u8(N * 2 * 210)
    xq, x = u8(Bd.q8_1_bytes(M, K)), f32(M, K)
    wp, we = u8(Bd.q6K_prep_bytes(N, K)), u8(Bd.q6K_exp_bytes(N, K))
    cases = [   # (call with a full-size output, call with an output one element short, entry reached)
        (lambda o: Bd.mmq_q4K_q8(w4, xq, M, N, K, o), f32(M * N), "mmq_q4K_q8"),
        (lambda o: Bd.mmq_q6K_q8(w6, xq, M, N, K, o), f32(M * N), "mmq_q6K_q8"),
        (lambda o: Bd.mmq_q4K_isums(w4, xq, M, N, K, o), i32(M * N * K // 32), "mmq_q4K_isums"),
        (lambda o: Bd.mmq_q6K_isums(w6, xq, M, N, K, o), i32(M * N * K // 16), "mmq_q6K_isums"),
        (lambda o: Bd.mmq_q6K_prep_q8(wp, xq, M, N, K, o), f32(M * N), "mmq_q6K_prep_q8"),
        (lambda o: Bd.mmq_q6K_prep_isums(wp, xq, M, N, K, o), i32(M * N * K // 16), "mmq_q6K_prep_isums"),
        (lambda o: Bd.mmq_q6K_exp_q8(we, xq, M, N, K, o), f32(M * N), "mmq_q6K_exp_q8"),
        (lambda o: Bd.mmq_q6K_exp_csums(we, xq, M, N, K, o), i32(M * N * K // 32), "mmq_q6K_exp_csums"),
        (lambda o: Bd.mmq_q4K(w4, x, N, y=o), f32(M * N), "mmq_q4K"),
        (lambda o: Bd.mmq_q4K(w4, x, N, xq_ws=o), u8(Bd.q8_1_bytes(M, K)), "mmq_q4K"),
        (lambda o: Bd.mmq_q6K(w6, x, N, y=o), f32(M * N), "mmq_q6K"),
        (lambda o: Bd.quantize_q8_1(x, o), u8(Bd.q8_1_bytes(M, K)), "quantize_q8_1"),
        (lambda o: Bd.q6K_prepare(w6, N, K, wp=o), u8(Bd.q6K_prep_bytes(N, K)), "q6K_prepare"),
        (lambda o: Bd.q6K_expand(w6, N, K, we=o), u8(Bd.q6K_exp_bytes(N, K)), "q6K_expand"),
        (lambda o: Bd.mmq_q4K_q8_sk(w4, xq, M, N, K, y=o), f32(M * N), "mmq_q4K_q8_sk"),
        (lambda o: Bd.mmq_q6K_exp_q8_sk(we, xq, M, N, K, y=o), f32(M * N), "mmq_q6K_exp_q8_sk"),
    ]
    for call, full, entry in cases:
        calls.clear()
        call(full)
        assert calls == [entry], (entry, calls)
        calls.clear()
        with pytest.raises(Bd.QPGError) as e:
            call(full[:-1])
        assert e.value.status == Bd.QPG_EINVAL, entry
        assert calls == [], f"{entry} reached the library with an undersized output"


def test_binding_rejects_undersized_splitk_workspace(recorded):
    import torch
    Bd, calls = recorded
    M, N, K = 64, 100, 1536                    # one tile, six super-blocks: two pieces
    nws = Bd.mmq_sk_bytes(M, N, K, "q4K")
    assert nws == 2 * M * N * 4
    w = torch.zeros(N * 6 * 144, dtype=torch.uint8)
    xq = torch.zeros(Bd.q8_1_bytes(M, K), dtype=torch.uint8)
    Bd.mmq_q4K_q8_sk(w, xq, M, N, K, ws=torch.zeros(nws // 4, dtype=torch.float32))
    assert calls == ["mmq_q4K_q8_sk"]
    calls.clear()
    with pytest.raises(Bd.QPGError):
        Bd.mmq_q4K_q8_sk(w, xq, M, N, K, ws=torch.zeros(nws // 4 - 1, dtype=torch.float32))
    assert calls == []


ESCRATCH = -5
NOALLOC_SCRATCH = 32 << 20


def test_noalloc_entry_rejects_before_enqueue(L):
    f = L.mmq_q4K_noalloc
    assert L.qpg_strerror(ESCRATCH)
    assert "#define QPG_NOALLOC_SCRATCH_BYTES (32u << 20)" in open(HEADER).read()
    K = 11008 - 11008 % 256 + 256                       # 11264: a multiple of 256
    fits = NOALLOC_SCRATCH // L.qpg_q8_1_bytes(1, K)
    assert L.qpg_q8_1_bytes(fits, K) <= NOALLOC_SCRATCH < L.qpg_q8_1_bytes(fits + 1, K)
    assert f(A16, A16, A16, fits + 1, 256, K, None) == ESCRATCH     # one token row too many
    assert f(None, A16, A16, 64, 256, 256, None) == EINVAL
    assert f(A16, None, A16, 64, 256, 256, None) == EINVAL
    assert f(A16, A16, None, 64, 256, 256, None) == EINVAL
    assert f(A16, A16, A16, 64, 256, 288, None) == EINVAL
    assert f(A8, A16, A16, 64, 256, 256, None) == EALIGN              # q4_K weights: 16 bytes
    assert f(A16, A8, A16, 64, 256, 256, None) == EALIGN              # x: 16 bytes
    assert f(A16, A16, A2, 64, 256, 256, None) == EALIGN              # y: 4 bytes
    if not _has_gpu():
        assert f(A16, A16, A16, fits, 256, K, None) == EDEVICE       # the largest shape passes validation
