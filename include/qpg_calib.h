/* libqpg_calib.so: measurement and probe helpers for the k-quant MMQ library (not part of the
 * GEMM path).
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

/* Compute-step ceiling of the q4_K MMQ kernel: its inner step with no memory traffic, no
 * barriers, no header decode and no min term. Per wave and step one v_mfma_i32_32x32x32_i8
 * onto the 1.5*2^23 constant, issued one step ahead, and the fold of the previous result
 * (e = fma(F, da, -1.5*2^23*da), y = fma(e, dsv, y) on its 16 registers: 32 f32 FMAs).
 *   mode 0: the MFMAs alone; 1: the fold alone (opaque operands); 2: the kernel's step;
 *   3: MFMAs and a fold that does not depend on them (do the two units run concurrently);
 *   4: each MFMA folded in its own step (no look-ahead); 5: the kernel's step with its
 *   operands (B, raw weights, d*sc, da pair) read from LDS as the kernel reads them;
 *   6: mode 5 with every LDS operand read one step ahead (double-buffered in registers);
 *   7: the kernel's step with its fold issued in groups of four independent FMAs.
 * waves_per_simd in {1, 2, 3, 4}: the launch holds exactly that many waves on every SIMD
 * (qpg_calib_step_blocks(w) workgroups of four waves, LDS sized so that w fit a CU; one
 * wave per SIMD is the situation of a short prompt's split, one workgroup per CU).
 * Every wave runs iters x 8 steps. out: device pointer to qpg_calib_step_blocks(w) * 4
 * uint64 values, 8-byte aligned, owned by the caller, written as for qpg_calib_mfma_i8.
 * Asynchronous on `stream`. Returns 0, -1 (bad mode, w, iters or null out), -2 (alignment),
 * -3 (launch error) or -4 (not gfx950). Nothing is allocated. */
int qpg_calib_step(int mode, int waves_per_simd, int64_t iters, uint64_t* out, void* stream);

/* Workgroups qpg_calib_step launches for waves_per_simd (CUs x w), 0 if w is outside
 * {1, 2, 3, 4} or the current device is not gfx950. */
int64_t qpg_calib_step_blocks(int waves_per_simd);

/* Matrix-instruction layout probe: one wave executes one instruction, lane l's source
 * registers read from a / b / c at lane-major offsets and its result registers written to d.
 *   kind 0: v_mfma_i32_32x32x32_i8   a, b: 64 x 16 bytes (int8x16), c, d: 64 x 16 int32
 *   kind 1: v_mfma_i32_32x32x16_i8   a, b: 64 x 8 bytes (int8x8),   c, d: 64 x 16 int32
 *   kind 2: v_mfma_f32_32x32x16_bf16 a, b: 64 x 8 bf16,             c, d: 64 x 16 f32
 * Device pointers owned by the caller; a and b 16-byte aligned (8 for kind 1), c and d 16.
 * Asynchronous on `stream`. Returns 0, -1 (null pointer or bad kind), -2 (alignment),
 * -3 (launch error) or -4 (not gfx950). */
int qpg_probe_mfma(int kind, const void* a, const void* b, const void* c, void* d, void* stream);

/* LDS-direct load probe: one wave issues one buffer_load_dword (width 4) or
 * buffer_load_dwordx4 (width 16) with the LDS flag, lane l reading at byte offset voff[l] of
 * the nbytes-byte buffer src (a buffer descriptor of that range: offsets past it read zeros),
 * into a 1 KiB LDS array pre-filled with 0xDEADBEEF, which is then copied to out (256
 * uint32). Device pointers owned by the caller: src 16-byte aligned, voff (64 int32) and out
 * 4-byte aligned. Asynchronous on `stream`. Returns 0, -1 (null pointer, width not 4 or 16,
 * nbytes outside [1, 2^30]), -2 (alignment), -3 (launch error) or -4 (not gfx950). */
int qpg_probe_lds_dma(int width, const void* src, int64_t nbytes, const int32_t* voff, uint32_t* out, void* stream);

/* v_permlane32_swap probe (the raw q6_K kernel exchanges operand pieces between the wave's
 * lane halves with it): one wave loads register a from in[0..63] and b from in[64..127]
 * (lane l: in[l], in[64 + l]), executes the swap, and writes a to out[0..63] and b to
 * out[64..127]. Device pointers owned by the caller, 4-byte aligned. Asynchronous on
 * `stream`. Returns 0, -1 (null pointer), -2 (alignment), -3 (launch error) or -4 (not
 * gfx950). */
int qpg_probe_permlane32_swap(const uint32_t* in, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
