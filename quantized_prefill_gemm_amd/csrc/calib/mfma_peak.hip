// Matrix-core peak probe for gfx950: chains of v_mfma_i32_32x32x32_i8 and nothing else
// (declared in include/qpg_calib.h). Used by bench.py to report the measured int8 peak and
// the shader clock next to the published figure.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../../include/qpg_calib.h"

namespace {

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef int int32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, uint64_t* out)
{
    const int tx = (int)threadIdx.x;
    int32x4 a = {tx, tx ^ 0x5A5A, 0x01020304, (int)blockIdx.x};
    const int32x4 b = {0x7F7F7F7F, tx * 3, 0x10203040, -tx};
    int32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
        }
        a[0] += 1;
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= c0[r] + c1[r] + c2[r] + c3[r];
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    // thread 0 reports (its checksum depends on every MFMA of the loop, so none is dropped)
    if (tx == 0) {
        out[4 * blockIdx.x + 0] = t1 - t0;
        out[4 * blockIdx.x + 1] = r1 - r0;
        out[4 * blockIdx.x + 2] = (uint64_t)(uint32_t)s;
        out[4 * blockIdx.x + 3] = 0;
    }
}

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -4;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return -4;
    const char* n = p.gcnArchName;
    return (n[0] == 'g' && n[1] == 'f' && n[2] == 'x' && n[3] == '9' && n[4] == '5' && n[5] == '0' &&
            (n[6] == 0 || n[6] == ':'))
               ? 0
               : -4;
}

}  // namespace

extern "C" int qpg_calib_mfma_i8(int64_t blocks, int64_t iters, uint64_t* out, void* stream)
{
    if (!out || blocks < 1 || blocks > 65536 || iters < 1 || iters > 10000000) return -1;
    if (((uintptr_t)out & 7) != 0) return -2;
    const int dv = check_device();
    if (dv != 0) return dv;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (int)iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
