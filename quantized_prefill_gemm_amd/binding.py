"""ctypes binding of libqpg.so: argument marshalling only.

Every step of the path runs in the HIP kernels of libqpg.so. torch provides device
memory and the stream (torch.cuda.current_stream()); nothing here computes. If the
library has not been built, the first call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqpg.so")

QPG_OK, QPG_EINVAL, QPG_EALIGN, QPG_EHIP, QPG_EDEVICE, QPG_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20     # QPG_NOALLOC_SCRATCH_BYTES of qpg.h


class QPGError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqpg.so once. Raises if it is missing (build with __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QPGError(QPG_EINVAL, f"libqpg.so not built at {LIB_PATH}")
        L = ctypes.CDLL(LIB_PATH)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.qpg_strerror.argtypes = [ctypes.c_int]
        L.qpg_strerror.restype = ctypes.c_char_p
        L.qpg_q8_1_bytes.argtypes = [I64, I64]
        L.qpg_q8_1_bytes.restype = ctypes.c_size_t
        L.quantize_q8_1.argtypes = [P, P, I64, I64, P]
        for f in (L.mmq_q4K, L.mmq_q6K):
            f.argtypes = [P, P, P, I64, I64, I64, P, P]
        L.mmq_q4K_noalloc.argtypes = [P, P, P, I64, I64, I64, P]
        L.mmq_q4K_noalloc.restype = ctypes.c_int
        for f in (L.mmq_q4K_q8, L.mmq_q6K_q8, L.mmq_q4K_isums, L.mmq_q6K_isums):
            f.argtypes = [P, P, P, I64, I64, I64, P]
        L.qpg_q6K_prep_bytes.argtypes = [I64, I64]
        L.qpg_q6K_prep_bytes.restype = ctypes.c_size_t
        L.q6K_prepare.argtypes = [P, P, I64, I64, P]
        for f in (L.mmq_q6K_prep_q8, L.mmq_q6K_prep_isums):
            f.argtypes = [P, P, P, I64, I64, I64, P]
        L.qpg_q6K_exp_bytes.argtypes = [I64, I64]
        L.qpg_q6K_exp_bytes.restype = ctypes.c_size_t
        L.q6K_expand.argtypes = [P, P, I64, I64, P]
        for f in (L.mmq_q6K_exp_q8, L.mmq_q6K_exp_csums):
            f.argtypes = [P, P, P, I64, I64, I64, P]
        L.qpg_mmq_sk_bytes.argtypes = [I64, I64, I64, ctypes.c_int]
        L.qpg_mmq_sk_bytes.restype = ctypes.c_size_t
        for f in (L.mmq_q4K_q8_sk, L.mmq_q6K_q8_sk, L.mmq_q6K_prep_q8_sk, L.mmq_q6K_exp_q8_sk):
            f.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
            f.restype = ctypes.c_int
        for f in (L.quantize_q8_1, L.mmq_q4K, L.mmq_q6K, L.mmq_q4K_q8, L.mmq_q6K_q8, L.mmq_q4K_isums,
                  L.mmq_q6K_isums, L.q6K_prepare, L.mmq_q6K_prep_q8, L.mmq_q6K_prep_isums, L.q6K_expand,
                  L.mmq_q6K_exp_q8, L.mmq_q6K_exp_csums):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


EXPORTS = ("qpg_strerror", "qpg_q8_1_bytes", "quantize_q8_1", "mmq_q4K", "mmq_q6K", "mmq_q4K_q8",
           "mmq_q6K_q8", "mmq_q4K_isums", "mmq_q6K_isums", "qpg_q6K_prep_bytes", "q6K_prepare",
           "mmq_q6K_prep_q8", "mmq_q6K_prep_isums", "qpg_q6K_exp_bytes", "q6K_expand", "mmq_q6K_exp_q8",
           "mmq_q6K_exp_csums", "qpg_mmq_sk_bytes", "mmq_q4K_q8_sk", "mmq_q6K_q8_sk", "mmq_q6K_prep_q8_sk",
           "mmq_q6K_exp_q8_sk", "mmq_q4K_noalloc")


def _check(rc: int, what: str):
    if rc != QPG_OK:
        raise QPGError(rc, f"{what}: {lib().qpg_strerror(rc).decode()}")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise QPGError(QPG_EINVAL, f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise QPGError(QPG_EINVAL, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise QPGError(QPG_EINVAL, f"{name} must be contiguous")


def _same_device(t: torch.Tensor, ref: torch.Tensor, name: str):
    if t.device != ref.device:
        raise QPGError(QPG_EINVAL, f"{name} is on {t.device}, the inputs on {ref.device}")


def _out(t: torch.Tensor, dtype, name: str, need: int, ref: torch.Tensor):
    """A caller-supplied output: device tensor of dtype, contiguous, on ref's device and
    holding at least `need` elements (the C ABI takes no output size, so an undersized
    buffer would be written past its end)."""
    _dev(t, dtype, name)
    _same_device(t, ref, name)
    if t.numel() < need:
        raise QPGError(QPG_EINVAL, f"{name} holds {t.numel()} elements, {need} needed")


def q8_1_bytes(M: int, K: int) -> int:
    return int(lib().qpg_q8_1_bytes(M, K))


def quantize_q8_1(x: torch.Tensor, xq: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x f32 [M, K] (device) -> uint8 q8_1 buffer of q8_1_bytes(M, K) bytes."""
    _dev(x, torch.float32, "x")
    M, K = x.shape
    nbytes = q8_1_bytes(M, K)
    if xq is None:
        xq = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _out(xq, torch.uint8, "xq", nbytes, x)
    _check(lib().quantize_q8_1(_ptr(x), _ptr(xq), M, K, _stream(stream)), "quantize_q8_1")
    return xq


def _wcheck(w: torch.Tensor, N: int, K: int, bytes_per_block: int):
    _dev(w, torch.uint8, "w")
    if w.numel() != N * (K // 256) * bytes_per_block:
        raise QPGError(QPG_EINVAL, "w size does not match N x K")


def _mmq(which: str, w, x, N, y, xq_ws, stream):
    _dev(x, torch.float32, "x")
    M, K = x.shape
    _wcheck(w, N, K, 144 if which == "q4K" else 210)
    _same_device(w, x, "w")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _out(y, torch.float32, "y", M * N, x)
    if xq_ws is None:
        xq_ws = torch.empty(max(q8_1_bytes(M, K), 1), dtype=torch.uint8, device=x.device)
    _out(xq_ws, torch.uint8, "xq_ws", q8_1_bytes(M, K), x)
    fn = lib().mmq_q4K if which == "q4K" else lib().mmq_q6K
    _check(fn(_ptr(w), _ptr(x), _ptr(y), M, N, K, _ptr(xq_ws), _stream(stream)), "mmq_" + which)
    return y


def mmq_q4K(w: torch.Tensor, x: torch.Tensor, N: int, y=None, xq_ws=None, stream=None) -> torch.Tensor:
    """Y f32 [M, N] = q4_K W [N, K] x q8_1(x)^T; w is the raw uint8 block buffer."""
    return _mmq("q4K", w, x, N, y, xq_ws, stream)


def mmq_q6K(w: torch.Tensor, x: torch.Tensor, N: int, y=None, xq_ws=None, stream=None) -> torch.Tensor:
    return _mmq("q6K", w, x, N, y, xq_ws, stream)


def mmq_q4K_noalloc(w: torch.Tensor, x: torch.Tensor, N: int, y: torch.Tensor, stream=None) -> torch.Tensor:
    """mmq_q4K with the q8_1 activations in the library's fixed per-device scratch: the C call
    allocates nothing (y is the caller's). Calls overlapping on one device race."""
    _dev(x, torch.float32, "x")
    M, K = x.shape
    _wcheck(w, N, K, 144)
    _same_device(w, x, "w")
    _out(y, torch.float32, "y", M * N, x)
    _check(lib().mmq_q4K_noalloc(_ptr(w), _ptr(x), _ptr(y), M, N, K, _stream(stream)), "mmq_q4K_noalloc")
    return y


def _mmq_q8(which: str, w, xq, M, N, K, out, stream, isums: bool):
    _dev(xq, torch.uint8, "xq")
    if xq.numel() < q8_1_bytes(M, K):
        raise QPGError(QPG_EINVAL, "xq too small")
    _wcheck(w, N, K, 144 if which == "q4K" else 210)
    _same_device(w, xq, "w")
    if isums:
        per = 32 if which == "q4K" else 16
        if out is None:
            out = torch.empty((M, N, K // per), dtype=torch.int32, device=xq.device)
        _out(out, torch.int32, "s", M * N * (K // per), xq)
        fn = lib().mmq_q4K_isums if which == "q4K" else lib().mmq_q6K_isums
    else:
        if out is None:
            out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
        _out(out, torch.float32, "y", M * N, xq)
        fn = lib().mmq_q4K_q8 if which == "q4K" else lib().mmq_q6K_q8
    _check(fn(_ptr(w), _ptr(xq), _ptr(out), M, N, K, _stream(stream)),
           ("mmq_%s_isums" if isums else "mmq_%s_q8") % which)
    return out


def mmq_q4K_q8(w, xq, M, N, K, y=None, stream=None):
    return _mmq_q8("q4K", w, xq, M, N, K, y, stream, False)


def mmq_q6K_q8(w, xq, M, N, K, y=None, stream=None):
    return _mmq_q8("q6K", w, xq, M, N, K, y, stream, False)


def mmq_q4K_isums(w, xq, M, N, K, s=None, stream=None):
    return _mmq_q8("q4K", w, xq, M, N, K, s, stream, True)


def mmq_q6K_isums(w, xq, M, N, K, s=None, stream=None):
    return _mmq_q8("q6K", w, xq, M, N, K, s, stream, True)


def q6K_prep_bytes(N: int, K: int) -> int:
    return int(lib().qpg_q6K_prep_bytes(N, K))


def q6K_prepare(w: torch.Tensor, N: int, K: int, wp=None, stream=None) -> torch.Tensor:
    """Raw q6_K blocks (uint8, N*(K/256)*210 bytes, device) -> prepared layout (uint8)."""
    _wcheck(w, N, K, 210)
    nbytes = q6K_prep_bytes(N, K)
    if nbytes == 0:
        raise QPGError(QPG_EINVAL, f"unsupported shape N={N} K={K}")
    if wp is None:
        wp = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _out(wp, torch.uint8, "wp", nbytes, w)
    _check(lib().q6K_prepare(_ptr(w), _ptr(wp), N, K, _stream(stream)), "q6K_prepare")
    return wp


def _mmq_prep(wp, xq, M, N, K, out, stream, isums: bool):
    _dev(xq, torch.uint8, "xq")
    if xq.numel() < q8_1_bytes(M, K):
        raise QPGError(QPG_EINVAL, "xq too small")
    _dev(wp, torch.uint8, "wp")
    _same_device(wp, xq, "wp")
    if wp.numel() < q6K_prep_bytes(N, K):
        raise QPGError(QPG_EINVAL, "wp too small")
    if isums:
        if out is None:
            out = torch.empty((M, N, K // 16), dtype=torch.int32, device=xq.device)
        _out(out, torch.int32, "s", M * N * (K // 16), xq)
        fn = lib().mmq_q6K_prep_isums
    else:
        if out is None:
            out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
        _out(out, torch.float32, "y", M * N, xq)
        fn = lib().mmq_q6K_prep_q8
    _check(fn(_ptr(wp), _ptr(xq), _ptr(out), M, N, K, _stream(stream)),
           "mmq_q6K_prep_isums" if isums else "mmq_q6K_prep_q8")
    return out


def mmq_q6K_prep_q8(wp, xq, M, N, K, y=None, stream=None):
    return _mmq_prep(wp, xq, M, N, K, y, stream, False)


def mmq_q6K_prep_isums(wp, xq, M, N, K, s=None, stream=None):
    return _mmq_prep(wp, xq, M, N, K, s, stream, True)


def q6K_exp_bytes(N: int, K: int) -> int:
    return int(lib().qpg_q6K_exp_bytes(N, K))


def q6K_expand(w: torch.Tensor, N: int, K: int, we=None, stream=None) -> torch.Tensor:
    """Raw q6_K blocks (uint8, N*(K/256)*210 bytes, device) -> expanded layout (uint8)."""
    _wcheck(w, N, K, 210)
    nbytes = q6K_exp_bytes(N, K)
    if nbytes == 0:
        raise QPGError(QPG_EINVAL, f"unsupported shape N={N} K={K}")
    if we is None:
        we = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _out(we, torch.uint8, "we", nbytes, w)
    _check(lib().q6K_expand(_ptr(w), _ptr(we), N, K, _stream(stream)), "q6K_expand")
    return we


def _mmq_exp(we, xq, M, N, K, out, stream, csums: bool):
    _dev(xq, torch.uint8, "xq")
    if xq.numel() < q8_1_bytes(M, K):
        raise QPGError(QPG_EINVAL, "xq too small")
    _dev(we, torch.uint8, "we")
    _same_device(we, xq, "we")
    if we.numel() < q6K_exp_bytes(N, K):
        raise QPGError(QPG_EINVAL, "we too small")
    if csums:
        if out is None:
            out = torch.empty((M, N, K // 32), dtype=torch.int32, device=xq.device)
        _out(out, torch.int32, "s", M * N * (K // 32), xq)
        fn = lib().mmq_q6K_exp_csums
    else:
        if out is None:
            out = torch.empty((M, N), dtype=torch.float32, device=xq.device)
        _out(out, torch.float32, "y", M * N, xq)
        fn = lib().mmq_q6K_exp_q8
    _check(fn(_ptr(we), _ptr(xq), _ptr(out), M, N, K, _stream(stream)),
           "mmq_q6K_exp_csums" if csums else "mmq_q6K_exp_q8")
    return out


def mmq_q6K_exp_q8(we, xq, M, N, K, y=None, stream=None):
    return _mmq_exp(we, xq, M, N, K, y, stream, False)


def mmq_q6K_exp_csums(we, xq, M, N, K, s=None, stream=None):
    return _mmq_exp(we, xq, M, N, K, s, stream, True)


# Weight forms of the K-split entry points (the form argument of qpg_mmq_sk_bytes).
SK_FORMS = {"q4K": 0, "q6K": 1, "q6K_prep": 2, "q6K_exp": 3}
_SK_FN = {"q4K": "mmq_q4K_q8_sk", "q6K": "mmq_q6K_q8_sk", "q6K_prep": "mmq_q6K_prep_q8_sk",
          "q6K_exp": "mmq_q6K_exp_q8_sk"}


def mmq_sk_bytes(M: int, N: int, K: int, form: str) -> int:
    """Workspace bytes of the K-split entry point for this shape (0: no split is made)."""
    return int(lib().qpg_mmq_sk_bytes(M, N, K, SK_FORMS[form]))


def _mmq_sk(form: str, w, xq, M, N, K, y, ws, stream):
    _dev(xq, torch.uint8, "xq")
    if xq.numel() < q8_1_bytes(M, K):
        raise QPGError(QPG_EINVAL, "xq too small")
    if form in ("q4K", "q6K"):
        _wcheck(w, N, K, 144 if form == "q4K" else 210)
    else:
        _dev(w, torch.uint8, "w")
        need = q6K_prep_bytes(N, K) if form == "q6K_prep" else q6K_exp_bytes(N, K)
        if w.numel() < need:
            raise QPGError(QPG_EINVAL, "w too small")
    _same_device(w, xq, "w")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _out(y, torch.float32, "y", M * N, xq)
    nws = mmq_sk_bytes(M, N, K, form)
    if ws is None and nws:
        ws = torch.empty(nws // 4, dtype=torch.float32, device=xq.device)
    if ws is not None:
        _out(ws, torch.float32, "ws", nws // 4, xq)
    wsb = 0 if ws is None else ws.numel() * 4
    _check(getattr(lib(), _SK_FN[form])(_ptr(w), _ptr(xq), _ptr(y), M, N, K, _ptr(ws), wsb, _stream(stream)),
           _SK_FN[form])
    return y


def mmq_q4K_q8_sk(w, xq, M, N, K, y=None, ws=None, stream=None):
    return _mmq_sk("q4K", w, xq, M, N, K, y, ws, stream)


def mmq_q6K_q8_sk(w, xq, M, N, K, y=None, ws=None, stream=None):
    return _mmq_sk("q6K", w, xq, M, N, K, y, ws, stream)


def mmq_q6K_prep_q8_sk(wp, xq, M, N, K, y=None, ws=None, stream=None):
    return _mmq_sk("q6K_prep", wp, xq, M, N, K, y, ws, stream)


def mmq_q6K_exp_q8_sk(we, xq, M, N, K, y=None, ws=None, stream=None):
    return _mmq_sk("q6K_exp", we, xq, M, N, K, y, ws, stream)
