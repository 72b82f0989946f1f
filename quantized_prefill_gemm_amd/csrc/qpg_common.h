// Internal definitions shared by the gfx950 kernels of libqpg (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qpg {

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef int int32x16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int QK_K = 256;        // weights per super-block
constexpr int QK8 = 32;          // values per q8_1 block (one "chunk" of K)
constexpr int Q4K_BYTES = 144;
constexpr int Q6K_BYTES = 210;



// Bits of the f32 value 1.5 * 2^23. An integer |v| < 2^22 added to these bits gives the
// bits of the f32 value 1.5*2^23 + v exactly (all such values share one exponent and
// unit spacing), so an int32 MFMA accumulating onto this constant delivers its integer
// sum already "converted": F = 1.5*2^23 + I, with no v_cvt instruction.
constexpr int MAGIC_BITS = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;

// C/D layout of the 32x32 MFMAs (verified by a lane probe on gfx950): lane l, register
// r holds row 8*(r>>2) + 4*(l>>5) + (r&3), column l&31. A and B operands: lane l holds
// row (A) / column (B) l&31 and the K-group l>>5 (16 bytes of int8, or 8 bf16).
__device__ __forceinline__ int c_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    _Float16 v;
    uint16_t b = (uint16_t)h;
    __builtin_memcpy(&v, &b, 2);
    return (float)v;
}

// Round-to-nearest-even f32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    uint32_t lsb = (u >> 16) & 1u;
    return (u + 0x7FFFu + lsb) >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace qpg

// Token-tile height of the q4_K kernel for a shape (the launcher and the split-K piece count
// both use this): 32 tokens (one 32-token sub-tile per wave) or 64. With t64 = the number of
// 64 x 128 tiles, 32-token tiles are taken when t64 <= 128 (too few tiles for 256 CUs: halving
// the tile doubles them and halves the token padding of a short prompt) or when M <= 256 and
// t64 > 256 (more workgroups per CU at four waves per SIMD); 64 otherwise. Measured on the 7B
// layer shapes (split-K entry, interleaved A/B): 4096 x 4096 at M = 16, 32, 64, 128, 256:
// 1.18, 1.23, 1.14, 1.23, 1.05x; 11008 x 4096 at M = 16, 32, 64, 256: 1.30, 1.28, 1.09, 1.08x,
// and 0.92x at M = 128 (172 tiles), which keeps 64.
inline int qpg_q4K_tile_m(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    const int64_t t64 = ((M + 63) / 64) * ((N + 127) / 128);
    return (t64 <= 128 || (M <= 256 && t64 > 256)) ? 32 : 64;
}

// Kernel launchers (defined in the .hip files; called by the C ABI layer after the
// arguments have been validated). They return hipGetLastError() of the launch.
hipError_t qpg_launch_quantize_q8_1(const float* x, void* xq, int64_t M, int64_t K, hipStream_t s);
// pieces > 1: K split over workgroups, y is then a [pieces][M][N] f32 workspace of partial
// sums (qpg_launch_splitk_reduce adds them); pieces = 1: y is the output.
hipError_t qpg_launch_mmq_q4K(const void* w, const void* xq, float* y, int32_t* isums,
                              int64_t M, int64_t N, int64_t K, int pieces, hipStream_t s);
hipError_t qpg_launch_mmq_q6K(const void* w, const void* xq, float* y, int32_t* isums,
                              int64_t M, int64_t N, int64_t K, int pieces, hipStream_t s);
// q6_K prepared layout: ceil(N/128) * (K/256) * 32 KiB (layout in mmq_q6k.hip)
hipError_t qpg_launch_q6K_prepare(const void* w, void* wp, int64_t N, int64_t K, hipStream_t s);
hipError_t qpg_launch_mmq_q6K_prep(const void* wp, const void* xq, float* y, int32_t* isums,
                                   int64_t M, int64_t N, int64_t K, int pieces, hipStream_t s);
// q6_K expanded layout: ceil(N/64) * (K/256) * 35,072 bytes (layout in mmq_q6k_exp.hip)
hipError_t qpg_launch_q6K_expand(const void* w, void* we, int64_t N, int64_t K, hipStream_t s);
hipError_t qpg_launch_mmq_q6K_exp(const void* we, const void* xq, float* y, int32_t* csums,
                                  int64_t M, int64_t N, int64_t K, int pieces, hipStream_t s);
// y[i] = sum over p < pieces of ws[p * MN + i], in piece order (deterministic).
hipError_t qpg_launch_splitk_reduce(const float* ws, float* y, int64_t MN, int pieces, hipStream_t s);
