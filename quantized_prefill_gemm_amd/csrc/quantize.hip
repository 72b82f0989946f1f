// q8_1 activation quantiser for gfx950.
//
// Per 32-value block ("chunk") of an f32 token row: amax = max|x|, d = amax/127,
// q = round(x * (1/d)) (ties away from zero), ssum = sum q, header word =
// fp16(d) | ssum << 16. The header packs the scale and the signed block sum in one
// 32-bit word per token and chunk, the form the MMQ kernels read ("r28 - Direction-A
// raw-nibble NB kernel", sec. 3.2 smem map; decoded as fp16 low half / int16 high half
// in "r14 - B fragments via ldmatrix", sec. 3.2(d)).
//
// HBM-bound: 4 B read per value, 1 + 1/8 B written. Each lane loads one float4 (16 B,
// fully coalesced: a wave reads 1 KiB contiguous), 8 lanes own one chunk, and the
// amax / sum reductions are 3 butterfly steps inside those 8 lanes. Chunks are indexed
// flat over (token, chunk), which is contiguous in both X and the q plane, so any
// K % 32 == 0 works with no per-row tail logic.
#include "qpg_common.h"

namespace qpg {

__device__ __forceinline__ float xor_max8(float v)
{
    v = fmaxf(v, __shfl_xor(v, 1, 8));
    v = fmaxf(v, __shfl_xor(v, 2, 8));
    v = fmaxf(v, __shfl_xor(v, 4, 8));
    return v;
}
__device__ __forceinline__ int xor_sum8(int v)
{
    v += __shfl_xor(v, 1, 8);
    v += __shfl_xor(v, 2, 8);
    v += __shfl_xor(v, 4, 8);
    return v;
}

// round(v) to int8, ties away from zero, saturated to [-127, 127]. v is infinite when
// 1/d overflowed (a block of tiny values): +-inf saturates, and NaN (x = 0 times inf)
// gives 0.
__device__ __forceinline__ int q8_round(float v)
{
    if (__builtin_isnan(v)) return 0;
    const float c = fminf(fmaxf(v, -127.0f), 127.0f);
    return (int)roundf(c);
}

__global__ void __launch_bounds__(256) quantize_q8_1_kernel(const float* __restrict__ x,
                                                            int8_t* __restrict__ qplane,
                                                            uint32_t* __restrict__ hdr,
                                                            int64_t nchunks)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one float4 each
    const int64_t chunk = gid >> 3;
    const int part = threadIdx.x & 7;
    const bool live = chunk < nchunks;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (live)
        v = *reinterpret_cast<const floatx4*>(x + chunk * QK8 + part * 4);
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = xor_max8(amax);
    const float d = __fdiv_rn(amax, 127.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    const int q0 = q8_round(v[0] * id), q1 = q8_round(v[1] * id);
    const int q2 = q8_round(v[2] * id), q3 = q8_round(v[3] * id);
    const int sum = xor_sum8(q0 + q1 + q2 + q3);
    if (live) {
        const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                                ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
        *reinterpret_cast<uint32_t*>(qplane + chunk * QK8 + part * 4) = packed;
        if (part == 0) {
            const _Float16 dh = (_Float16)d;                     // round to nearest even
            uint16_t dbits;
            __builtin_memcpy(&dbits, &dh, 2);
            hdr[chunk] = (uint32_t)dbits | ((uint32_t)(uint16_t)(int16_t)sum << 16);
        }
    }
}

}  // namespace qpg

hipError_t qpg_launch_quantize_q8_1(const float* x, void* xq, int64_t M, int64_t K, hipStream_t s)
{
    const int64_t nchunks = M * (K / qpg::QK8);
    int8_t* qplane = static_cast<int8_t*>(xq);
    uint32_t* hdr = reinterpret_cast<uint32_t*>(qplane + M * K);
    const int64_t threads = nchunks * 8;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(qpg::quantize_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, qplane, hdr,
                       nchunks);
    return hipGetLastError();
}
