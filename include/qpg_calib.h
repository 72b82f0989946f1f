/* libqpg_calib.so: measurement helper for the k-quant MMQ library (not part of the GEMM path).
 *
 * The int8 MFMA roofline of the MMQ kernels is priced against the published dense peak of
 * the device; this library measures the peak the matrix cores actually reach, and the
 * shader clock they reach it at, with a kernel that does nothing but chains of
 * v_mfma_i32_32x32x32_i8 (32x32x32 int8 products into int32, the instruction the q4_K
 * kernel uses).
 */
#ifndef QPG_CALIB_H
#define QPG_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `blocks` workgroups of 256 threads (4 waves); every wave issues `iters` x 16
 * v_mfma_i32_32x32x32_i8 on four independent accumulators (65,536 int8 operations each).
 * out: device pointer to blocks * 4 uint64 values, 8-byte aligned, owned by the caller:
 *   out[4b + 0] = shader-clock ticks (s_memtime) of workgroup b's wave 0 over its loop,
 *   out[4b + 1] = ticks of the 100 MHz constant clock (s_memrealtime) over the same loop,
 *   out[4b + 2] = a checksum of the accumulators (keeps the products live), out[4b + 3] = 0.
 * Asynchronous on `stream` (a hipStream_t, NULL = default stream).
 * Returns 0, -1 (QPG_EINVAL: null out, blocks outside [1, 65536], iters outside [1, 10^7]),
 * -2 (QPG_EALIGN), -3 (QPG_EHIP: launch error) or -4 (QPG_EDEVICE: current device is not
 * gfx950). Nothing is allocated. */
int qpg_calib_mfma_i8(int64_t blocks, int64_t iters, uint64_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
