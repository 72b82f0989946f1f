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
// fully coalesced: a wave reads 1 KiB contiguous) per slice, 8 lanes own one chunk, and the
// amax / sum reductions are 3 DPP steps inside those 8 lanes. Chunks are indexed
// flat over (token, chunk), which is contiguous in both X and the q plane, so any
// K % 32 == 0 works with no per-row tail logic.
#include "qpg_common.h"

namespace qpg {

// Reductions over the 8 lanes of a chunk by DPP lane moves (no LDS round trip): the two
// quad_perm exchanges (lane ^ 1, lane ^ 2) leave every lane of a quad with the quad's value,
// and row_half_mirror (lane i <-> 7 - i inside each group of 8) then brings the other quad's.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;            // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;            // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;    // row_half_mirror

__device__ __forceinline__ float max8(float v)
{
    v = fmaxf(v, __int_as_float(dpp_move<DPP_XOR1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<DPP_XOR2>(__float_as_int(v))));
    return fmaxf(v, __int_as_float(dpp_move<DPP_HALF_MIRROR>(__float_as_int(v))));
}
__device__ __forceinline__ int sum8(int v)
{
    v += dpp_move<DPP_XOR1>(v);
    v += dpp_move<DPP_XOR2>(v);
    return v + dpp_move<DPP_HALF_MIRROR>(v);
}

// round(v) to int8, ties away from zero, saturated to [-127, 127], without branches. v is
// infinite when 1/d overflowed (a block of tiny values): +-inf saturates, and NaN (x = 0
// times inf) gives 0. For c in [-127, 127], c + copysign(0.5 - 2^-25, c) rounded to f32 and
// truncated is c rounded half away from zero: below a half the sum stays under the next
// integer by at least half a unit in its last place, and at or above a half it reaches it
// (checked for every f32 in the range).
__device__ __forceinline__ int q8_round(float v)
{
    const float c = fminf(fmaxf(v, -127.0f), 127.0f);
    const int q = (int)(c + __builtin_copysignf(0.49999997f, c));     // conversion truncates
    return v == v ? q : 0;
}

// Each workgroup covers SLICES consecutive 4 KiB slices of X (256 lanes x one float4); a
// lane issues the loads of all its slices before it computes, which keeps more bytes in
// flight per wave than one float4 would.
constexpr int SLICES = 2;

__global__ void __launch_bounds__(256) quantize_q8_1_kernel(const float* __restrict__ x,
                                                            int8_t* __restrict__ qplane,
                                                            uint32_t* __restrict__ hdr,
                                                            int64_t nchunks)
{
    const int part = threadIdx.x & 7;
    floatx4 v[SLICES];
    int64_t chunk[SLICES];
#pragma unroll
    for (int u = 0; u < SLICES; ++u) {
        const int64_t gid = ((int64_t)blockIdx.x * SLICES + u) * 256 + threadIdx.x;   // one float4 each
        chunk[u] = gid >> 3;
        v[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (chunk[u] < nchunks) v[u] = *reinterpret_cast<const floatx4*>(x + chunk[u] * QK8 + part * 4);
    }
#pragma unroll
    for (int u = 0; u < SLICES; ++u) {
        float amax = fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3])));
        amax = max8(amax);
        const float d = __fdiv_rn(amax, 127.0f);
        const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
        const int q0 = q8_round(v[u][0] * id), q1 = q8_round(v[u][1] * id);
        const int q2 = q8_round(v[u][2] * id), q3 = q8_round(v[u][3] * id);
        const int sum = sum8(q0 + q1 + q2 + q3);
        if (chunk[u] < nchunks) {
            const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                                    ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
            *reinterpret_cast<uint32_t*>(qplane + chunk[u] * QK8 + part * 4) = packed;
            if (part == 0) {
                const _Float16 dh = (_Float16)d;                 // round to nearest even
                uint16_t dbits;
                __builtin_memcpy(&dbits, &dh, 2);
                hdr[chunk[u]] = (uint32_t)dbits | ((uint32_t)(uint16_t)(int16_t)sum << 16);
            }
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
    const int64_t blocks = (threads + 256 * qpg::SLICES - 1) / (256 * qpg::SLICES);
    hipLaunchKernelGGL(qpg::quantize_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, qplane, hdr,
                       nchunks);
    return hipGetLastError();
}
