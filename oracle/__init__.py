"""CPU oracle of the k-quant prefill GEMM. Test infrastructure only (see oracle.c)."""
