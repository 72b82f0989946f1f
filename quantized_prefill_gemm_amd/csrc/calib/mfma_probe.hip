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

// ---- LDS-direct load probe: one wave issues one buffer_load_dword / _dwordx4 with the LDS
// flag from host-chosen per-lane source offsets into a buffer of nbytes bytes; the LDS
// contents (pre-filled with 0xDEADBEEF) are then copied out. Shows where lane L's bytes land
// (4 L / 16 L), that any per-lane source offset is honoured (permutations, offsets that are
// not multiples of the load size), and that offsets past the buffer read as zeros.
namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <int WIDTH>
__global__ void __launch_bounds__(64) probe_lds_dma_kernel(const uint8_t* src, int nbytes, const int* voff, uint32_t* out)
{
    __shared__ uint32_t buf[256];
    const int l = (int)threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[4 * l + i] = 0xDEADBEEFu;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, nbytes, 0x00020000);
    const unsigned la = (unsigned)(uintptr_t)(lds_void*)buf;
    const int v = voff[l];
    if constexpr (WIDTH == 16)
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(v), "s"(r), "{m0}"(la) : "memory");
    else
        asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(v), "s"(r), "{m0}"(la) : "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): the load has written LDS
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) out[4 * l + i] = buf[4 * l + i];
}

}  // namespace

extern "C" int qpg_probe_lds_dma(int width, const void* src, int64_t nbytes, const int32_t* voff, uint32_t* out,
                                 void* stream)
{
    if (!src || !voff || !out || (width != 4 && width != 16) || nbytes < 1 || nbytes > (1 << 30)) return -1;
    if (((uintptr_t)src & 15) || ((uintptr_t)voff & 3) || ((uintptr_t)out & 3)) return -2;
    if (!is_gfx950()) return -4;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (width == 16)
        hipLaunchKernelGGL(probe_lds_dma_kernel<16>, dim3(1), dim3(64), 0, s, static_cast<const uint8_t*>(src),
                           (int)nbytes, voff, out);
    else
        hipLaunchKernelGGL(probe_lds_dma_kernel<4>, dim3(1), dim3(64), 0, s, static_cast<const uint8_t*>(src),
                           (int)nbytes, voff, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ---- v_permlane32_swap probe: one wave swaps register a's upper 32 lanes with register b's
// lower 32 lanes; in = a then b (64 words each), out = the two registers afterwards.
namespace {

__global__ void __launch_bounds__(64) probe_permlane32_swap_kernel(const uint32_t* in, uint32_t* out)
{
    const int l = (int)threadIdx.x;
    const auto r = __builtin_amdgcn_permlane32_swap(in[l], in[64 + l], false, false);
    out[l] = r[0];
    out[64 + l] = r[1];
}

}  // namespace

extern "C" int qpg_probe_permlane32_swap(const uint32_t* in, uint32_t* out, void* stream)
{
    if (!in || !out) return -1;
    if (((uintptr_t)in | (uintptr_t)out) & 3) return -2;
    if (!is_gfx950()) return -4;
    hipLaunchKernelGGL(probe_permlane32_swap_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), in, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
