// Sum of the K-split partial tiles: y[i] = ws[0][i] + ws[1][i] + ... in piece order, so the
// result does not depend on which workgroup finished first. Four floats per thread when the
// plane is a whole number of float4 (it is whenever N % 4 == 0), else one.
#include "qpg_common.h"

namespace qpg {

__global__ void __launch_bounds__(256) splitk_reduce4_kernel(const floatx4* __restrict__ ws, floatx4* __restrict__ y,
                                                            int64_t n4, int pieces)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    floatx4 acc = ws[i];
    for (int p = 1; p < pieces; ++p) {
        const floatx4 v = ws[(int64_t)p * n4 + i];
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
    }
    y[i] = acc;
}

__global__ void __launch_bounds__(256) splitk_reduce1_kernel(const float* __restrict__ ws, float* __restrict__ y,
                                                            int64_t n, int pieces)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float acc = ws[i];
    for (int p = 1; p < pieces; ++p) acc += ws[(int64_t)p * n + i];
    y[i] = acc;
}

}  // namespace qpg

hipError_t qpg_launch_splitk_reduce(const float* ws, float* y, int64_t MN, int pieces, hipStream_t s)
{
    const bool vec = (MN & 3) == 0 && (((uintptr_t)ws | (uintptr_t)y) & 15) == 0;
    if (vec) {
        const int64_t n4 = MN / 4;
        hipLaunchKernelGGL(qpg::splitk_reduce4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const qpg::floatx4*>(ws), reinterpret_cast<qpg::floatx4*>(y), n4, pieces);
    } else {
        hipLaunchKernelGGL(qpg::splitk_reduce1_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, ws, y, MN,
                           pieces);
    }
    return hipGetLastError();
}
