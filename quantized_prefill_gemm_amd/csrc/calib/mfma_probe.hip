// Operand-layout probe of the gfx950 matrix instructions the MMQ kernels use (declared in
// include/qpg_calib.h): one wave executes one instruction with every lane's source registers
// taken from host-chosen bytes and its result registers written back, so a test can map each
// lane / register to matrix coordinates, and check exact accumulation, against a plain
// matrix product on the host.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../../include/qpg_calib.h"

namespace {

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef int int32x16 __attribute__((ext_vector_type(16)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// lane-major operands: a, b 16 bytes per lane (8 for the K = 16 int8 form), c and d 64 bytes
__global__ void __launch_bounds__(64) probe_i8_k32(const int32x4* a, const int32x4* b, const int32x16* c, int32x16* d)
{
    const int l = (int)threadIdx.x;
    d[l] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[l], b[l], c[l], 0, 0, 0);
}

__global__ void __launch_bounds__(64) probe_i8_k16(const long* a, const long* b, const int32x16* c, int32x16* d)
{
    const int l = (int)threadIdx.x;
    d[l] = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[l], b[l], c[l], 0, 0, 0);
}

__global__ void __launch_bounds__(64) probe_bf16_k16(const bf16x8* a, const bf16x8* b, const floatx16* c, floatx16* d)
{
    const int l = (int)threadIdx.x;
    d[l] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[l], b[l], c[l], 0, 0, 0);
}

bool is_gfx950()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
    const char* n = p.gcnArchName;
    return n[0] == 'g' && n[1] == 'f' && n[2] == 'x' && n[3] == '9' && n[4] == '5' && n[5] == '0' &&
           (n[6] == 0 || n[6] == ':');
}

}  // namespace

extern "C" int qpg_probe_mfma(int kind, const void* a, const void* b, const void* c, void* d, void* stream)
{
    if (!a || !b || !c || !d || kind < 0 || kind > 2) return -1;
    const uintptr_t al = kind == 1 ? 8 : 16;
    if (((uintptr_t)a | (uintptr_t)b) & (al - 1) || ((uintptr_t)c | (uintptr_t)d) & 15) return -2;
    if (!is_gfx950()) return -4;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (kind) {
    case 0:
        hipLaunchKernelGGL(probe_i8_k32, dim3(1), dim3(64), 0, s, static_cast<const int32x4*>(a),
                           static_cast<const int32x4*>(b), static_cast<const int32x16*>(c), static_cast<int32x16*>(d));
        break;
    case 1:
        hipLaunchKernelGGL(probe_i8_k16, dim3(1), dim3(64), 0, s, static_cast<const long*>(a),
                           static_cast<const long*>(b), static_cast<const int32x16*>(c), static_cast<int32x16*>(d));
        break;
    default:
        hipLaunchKernelGGL(probe_bf16_k16, dim3(1), dim3(64), 0, s, static_cast<const bf16x8*>(a),
                           static_cast<const bf16x8*>(b), static_cast<const floatx16*>(c), static_cast<floatx16*>(d));
        break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
