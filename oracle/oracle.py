"""ctypes wrapper of the CPU oracle (oracle.c). TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
module. The product path (quantized_prefill_gemm_amd) never imports it and shares no
code with it. All arrays are numpy, host memory.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
           "-o", _LIB, _SRC, "-lm", "-lpthread"]


def build() -> str:
    """Compile oracle.c into liboracle.so (plain gcc, host only)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.qo_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.qo_f16_to_f64.restype = ctypes.c_double
        L.qo_f32_to_f16.argtypes = [ctypes.c_float]
        L.qo_f32_to_f16.restype = ctypes.c_uint16
        L.qo_quantize_q8_1.argtypes = [P, I64, I64, P, P, P]
        L.qo_decode_q4K.argtypes = [P, P, P, P, P, P]
        L.qo_decode_q6K.argtypes = [P, P, P, P]
        L.qo_dequant_q4K.argtypes = [P, I64, I64, P]
        L.qo_dequant_q6K.argtypes = [P, I64, I64, P]
        for f in (L.qo_isums_q4K, L.qo_isums_q6K):
            f.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int]
        for f in (L.qo_mmq_q4K, L.qo_mmq_q6K):
            f.argtypes = [P, P, P, P, I64, I64, I64, P, ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, min(64, len(os.sched_getaffinity(0))))


def f16_to_f64(h: int) -> float:
    return lib().qo_f16_to_f64(int(h))


def f32_to_f16(x: float) -> int:
    return int(lib().qo_f32_to_f16(float(x)))


def quantize_q8_1(x: np.ndarray):
    """x f32 [M, K] -> (q int8 [M, K], dh uint16 [M, K/32] fp16 bits, ssum int16 [M, K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    dh = np.empty((M, K // 32), np.uint16)
    ss = np.empty((M, K // 32), np.int16)
    rc = lib().qo_quantize_q8_1(_p(x), M, K, _p(q), _p(dh), _p(ss))
    if rc:
        raise ValueError("qo_quantize_q8_1 failed")
    return q, dh, ss


def decode_q4K(block: np.ndarray):
    """One 144-byte block -> (d, dmin, sc[8], m[8], nib[256])."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == 144
    d = ctypes.c_double()
    dm = ctypes.c_double()
    sc = np.empty(8, np.int32)
    m = np.empty(8, np.int32)
    nib = np.empty(256, np.int32)
    lib().qo_decode_q4K(_p(b), ctypes.byref(d), ctypes.byref(dm), _p(sc), _p(m), _p(nib))
    return d.value, dm.value, sc, m, nib


def decode_q6K(block: np.ndarray):
    """One 210-byte block -> (d, sc[16], v[256])."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == 210
    d = ctypes.c_double()
    sc = np.empty(16, np.int32)
    v = np.empty(256, np.int32)
    lib().qo_decode_q6K(_p(b), ctypes.byref(d), _p(sc), _p(v))
    return d.value, sc, v


def dequant(wtype: str, w: np.ndarray, K: int) -> np.ndarray:
    """Weights [N, blocks] -> fp64 [N, K]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    N = w.shape[0]
    out = np.empty((N, K), np.float64)
    f = lib().qo_dequant_q4K if wtype == "q4_K" else lib().qo_dequant_q6K
    if f(_p(w), N, K, _p(out)):
        raise ValueError("dequant failed")
    return out


def isums(wtype: str, w: np.ndarray, q: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """Exact integer sub-block sums: int32 [M, N, K/32] (q4_K) or [M, N, K/16] (q6_K)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = q.shape
    N = w.shape[0]
    per = 32 if wtype == "q4_K" else 16
    s = np.empty((M, N, K // per), np.int32)
    f = lib().qo_isums_q4K if wtype == "q4_K" else lib().qo_isums_q6K
    if f(_p(w), _p(q), M, N, K, _p(s), nthreads or default_threads()):
        raise ValueError("isums failed")
    return s


def q6K_chunk_sums(w: np.ndarray, q: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """Scale-weighted integer sums of q6_K per 32-wide chunk: int32 [M, N, K/32] with
    C[i, j, c] = sum over k in chunk c of sc[j, k/16] * v[j, k] * q[i, k] — the two 16-wide
    sub-block sums J of the chunk, each times its int8 scale (the fold of q6_K without the
    f32 factors da and d). |C| <= 2 * 128 * 16 * 32 * 127 < 2^31."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    J = isums("q6_K", w, q, nthreads).astype(np.int64)           # [M, N, K/16]
    N, K = w.shape[0], q.shape[1]
    nsb = K // 256
    sc = w.reshape(N, nsb, 210)[:, :, 192:208].view(np.int8).astype(np.int64).reshape(N, K // 16)
    C = J[:, :, 0::2] * sc[None, :, 0::2] + J[:, :, 1::2] * sc[None, :, 1::2]
    return C.astype(np.int32)


def mmq_q8(wtype: str, w: np.ndarray, q: np.ndarray, dh: np.ndarray, ss: np.ndarray,
           nthreads: int | None = None) -> np.ndarray:
    """fp64 [M, N] = fold of the exact integer sums (q8_1 activations given)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    dh = np.ascontiguousarray(dh, dtype=np.uint16)
    ss = np.ascontiguousarray(ss, dtype=np.int16)
    M, K = q.shape
    N = w.shape[0]
    y = np.empty((M, N), np.float64)
    f = lib().qo_mmq_q4K if wtype == "q4_K" else lib().qo_mmq_q6K
    if f(_p(w), _p(q), _p(dh), _p(ss), M, N, K, _p(y), nthreads or default_threads()):
        raise ValueError("mmq failed")
    return y


def mmq(wtype: str, w: np.ndarray, x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """fp64 [M, N] for f32 activations x: quantize_q8_1 then the exact fold."""
    q, dh, ss = quantize_q8_1(x)
    return mmq_q8(wtype, w, q, dh, ss, nthreads)


def dequant_activations(q: np.ndarray, dh: np.ndarray) -> np.ndarray:
    """fp64 [M, K]: each q8_1 value times its block's fp16 scale."""
    M, K = q.shape
    da = np.vectorize(f16_to_f64, otypes=[np.float64])(dh)
    return q.astype(np.float64) * np.repeat(da, 32, axis=1)


def brute_force(wtype: str, w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Plain definition: dequant(W) . dequant(q8_1(X))^T in fp64 (tiny shapes only)."""
    q, dh, _ = quantize_q8_1(x)
    K = q.shape[1]
    return dequant_activations(q, dh) @ dequant(wtype, w, K).T
