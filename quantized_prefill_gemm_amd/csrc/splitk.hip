// Sum of the K-split partial tiles: y[i] = ws[0][i] + ws[1][i] + ... in piece order, so the
// result does not depend on which workgroup finished first. Four floats per thread when the
// plane is a whole number of float4 (it is whenever N % 4 == 0), else one. The piece count is
// a template parameter: every partial of a thread is loaded before the first add, so a call
// waits for one memory round trip instead of one per piece.
#include "qpg_common.h"

namespace qpg {

template <int P>
__global__ void __launch_bounds__(256) splitk_reduce4_kernel(const floatx4* __restrict__ ws, floatx4* __restrict__ y,
                                                            int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    floatx4 v[P];
#pragma unroll
    for (int p = 0; p < P; ++p) v[p] = ws[(int64_t)p * n4 + i];
    floatx4 acc = v[0];
#pragma unroll
    for (int p = 1; p < P; ++p) {
        acc[0] += v[p][0];
        acc[1] += v[p][1];
        acc[2] += v[p][2];
        acc[3] += v[p][3];
    }
    y[i] = acc;
}

template <int P>
__global__ void __launch_bounds__(256) splitk_reduce1_kernel(const float* __restrict__ ws, float* __restrict__ y,
                                                            int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float v[P];
#pragma unroll
    for (int p = 0; p < P; ++p) v[p] = ws[(int64_t)p * n + i];
    float acc = v[0];
#pragma unroll
    for (int p = 1; p < P; ++p) acc += v[p];
    y[i] = acc;
}

template <int P>
hipError_t launch_reduce(const float* ws, float* y, int64_t MN, hipStream_t s)
{
    const bool vec = (MN & 3) == 0 && (((uintptr_t)ws | (uintptr_t)y) & 15) == 0;
    if (vec) {
        const int64_t n4 = MN / 4;
        hipLaunchKernelGGL(splitk_reduce4_kernel<P>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const floatx4*>(ws), reinterpret_cast<floatx4*>(y), n4);
    } else {
        hipLaunchKernelGGL(splitk_reduce1_kernel<P>, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, ws, y, MN);
    }
    return hipGetLastError();
}

}  // namespace qpg

// pieces in 2..8 (the K-split entry points' range); hipErrorInvalidValue otherwise
hipError_t qpg_launch_splitk_reduce(const float* ws, float* y, int64_t MN, int pieces, hipStream_t s)
{
    switch (pieces) {
    case 2: return qpg::launch_reduce<2>(ws, y, MN, s);
    case 3: return qpg::launch_reduce<3>(ws, y, MN, s);
    case 4: return qpg::launch_reduce<4>(ws, y, MN, s);
    case 5: return qpg::launch_reduce<5>(ws, y, MN, s);
    case 6: return qpg::launch_reduce<6>(ws, y, MN, s);
    case 7: return qpg::launch_reduce<7>(ws, y, MN, s);
    case 8: return qpg::launch_reduce<8>(ws, y, MN, s);
    default: return hipErrorInvalidValue;
    }
}
