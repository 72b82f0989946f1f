"""MI355X-native k-quant prefill GEMM: q4_K / q6_K weights x q8_1 activations on gfx950.

The compute path is the HIP library libqpg.so (C ABI declared in include/qpg.h); the
Python names below are thin ctypes marshalling over it. Importing the package does not
load the library; the first call does, and fails loudly if it has not been built.
"""
from . import inputs  # noqa: F401  (seeded synthetic inputs; no compute)

__all__ = ["inputs", "q8_1_bytes", "quantize_q8_1", "mmq_q4K", "mmq_q6K", "mmq_q4K_q8", "mmq_q6K_q8",
           "mmq_q4K_isums", "mmq_q6K_isums", "q6K_prep_bytes", "q6K_prepare", "mmq_q6K_prep_q8",
           "mmq_q6K_prep_isums", "q6K_exp_bytes", "q6K_expand", "mmq_q6K_exp_q8", "mmq_q6K_exp_csums",
           "mmq_sk_bytes", "mmq_q4K_q8_sk", "mmq_q6K_q8_sk", "mmq_q6K_prep_q8_sk", "mmq_q6K_exp_q8_sk", "QPGError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
