// Compute-step ceiling probe for gfx950 (declared in include/qpg_calib.h).
//
// The q4_K MMQ kernel's inner step, with nothing else: per wave and step, one
// v_mfma_i32_32x32x32_i8 onto the bits of 1.5*2^23 (issued one step ahead of its use), then
// the fold of the previous step's 16 accumulator registers -- e = fma(F, da, -1.5*2^23*da),
// y = fma(e, dsv, y): 32 f32 FMAs -- into one of two token sub-tiles' accumulators. No
// global or LDS traffic, no barriers, no header decode, no min term: the rate this runs at
// is the ceiling of the kernel's arithmetic at a given number of waves per SIMD.
//
// Variants isolate the two units:
//   mode 0  the MFMAs alone (same issue pattern, results only kept live),
//   mode 1  the fold alone (its F operands made opaque per step instead of MFMA results),
//   mode 2  the kernel's step: MFMA one step ahead, fold of the previous result,
//   mode 3  MFMA and fold with no dependency between them (the fold reads opaque values):
//           shows whether the matrix core and the VALU run concurrently at all,
//   mode 4  each step's MFMA folded in the same step (no look-ahead: half the result
//           registers; other waves on the SIMD have to cover the MFMA's latency),
//   mode 5  the kernel's step with its operands read from LDS as the kernel reads them: per
//           step the 16-byte B operand and the (da, -1.5*2^23*da) pair, every second step
//           the 16-byte raw weight word (unpacked to nibbles) and the 16 d*sc values,
//   mode 6  mode 5 with every LDS operand read one step before the step that uses it
//           (double-buffered in registers), so no read is waited for in its own step,
//   mode 7  the kernel's step (as mode 2) with the fold issued in groups of four: four
//           independent first FMAs, then the four accumulating ones.
// Occupancy is fixed by the launch: 256 * W workgroups of four waves, each holding
// 160 KiB / W of LDS (touched once), so every CU runs exactly W workgroups and each SIMD
// W waves.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../../include/qpg_calib.h"

namespace {

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef int int32x16 __attribute__((ext_vector_type(16)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMagicBits = 0x4B400000;          // bits of the f32 value 1.5 * 2^23
constexpr float kMagic = 12582912.0f;

template <int W>
struct LdsCap {
    static constexpr int bytes = (160 * 1024 / W) & ~1023;
};

template <int MODE, int W>
__global__ void __launch_bounds__(256, W) step_kernel(int iters, uint64_t* out)
{
    __shared__ int cap[LdsCap<W>::bytes / 4];
    const int tx = (int)threadIdx.x, lane = tx & 63;
    // operand area of mode 5 (16 KiB): small finite floats, any bytes for the int8 operands
    for (int i = tx; i < 4096; i += 256) cap[i] = __float_as_int(0.0009765625f * (float)(1 + (i & 7)));
    __syncthreads();
    int32x4 a = {lane * 0x01010101, 0x0F0E0D0C, 0x07060504 ^ lane, (int)blockIdx.x};
    const int32x4 b = {0x7F017F01, tx * 3, 0x10203040, -tx};
    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = kMagicBits;
    // fold terms: da is an exact f16 value, c0 = -1.5*2^23*da exact, dsv per register
    const float da = 0.0078125f * (float)(1 + (lane & 7)), c0 = -kMagic * da;
    float dal = da, c0l = c0;       // modes 5 and 6 read them from LDS every step
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) dsv[r] = 0.001f * (float)(r + 1 + (lane & 3));
    // mode 6: operands read one step ahead, double-buffered
    int32x4 ab[2] = {a, a}, bb[2] = {b, b};
    float dsb[2][16];
    int2 adb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) dsb[0][r] = dsb[1][r] = dsv[r];
    adb[0] = adb[1] = int2{__float_as_int(da), __float_as_int(c0)};
    floatx16 y[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[t][r] = 0.0f;
    int32x16 F[2];
    F[0] = magic;
    F[1] = magic;
    F[0][0] += lane;
    int32x16 opaque = F[0];

    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (MODE != 1 && MODE != 4) F[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, magic, 0, 0, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            asm volatile("" : "+v"(magic));
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MODE == 6) {
                // this step: MFMA k+1 with the B operand read last step, fold k with the d*sc and
                // (da, c0) read last step; then the reads for step k+1 (B of MFMA k+2)
                __builtin_amdgcn_sched_barrier(0);
                F[(k + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ab[k & 1], bb[k & 1], magic, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) dsv[r] = dsb[k & 1][r];
                dal = __int_as_float(adb[k & 1].x);
                c0l = __int_as_float(adb[k & 1].y);
                const int kn = k + 1;
                bb[kn & 1] = *reinterpret_cast<const int32x4*>(&cap[((kn & 3) * 1024 + lane * 16) / 4]);
                if ((kn & 1) == 0)
                    ab[kn & 1] = *reinterpret_cast<const int32x4*>(&cap[(4096 + (kn & 2) * 512 + lane * 16) / 4]) & 0x0F0F0F0F;
                else
                    ab[kn & 1] = ab[k & 1];
                if ((kn & 1) == 0) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int32x4 d4 = *reinterpret_cast<const int32x4*>(&cap[(8192 + ((kn >> 1) & 3) * 512 + (lane >> 5) * 64 + q4 * 16) / 4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) dsb[kn & 1][4 * q4 + e] = __int_as_float(d4[e]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) dsb[kn & 1][r] = dsb[k & 1][r];
                }
                adb[kn & 1] = *reinterpret_cast<const int2*>(&cap[(12288 + (kn & 7) * 256 + (lane & 31) * 8) / 4]);
            } else if constexpr (MODE == 5) {
                // operands of this step from LDS: B of the next MFMA, raw weights every other
                // step, then this fold's d*sc (every other step) and (da, c0)
                const int32x4 bn = *reinterpret_cast<const int32x4*>(&cap[((k & 3) * 1024 + lane * 16) / 4]);
                if ((k & 1) == 0) {
                    const int32x4 raw = *reinterpret_cast<const int32x4*>(&cap[(4096 + (k & 2) * 512 + lane * 16) / 4]);
                    a = raw & 0x0F0F0F0F;
                }
                if ((k & 1) == 0) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int32x4 d4 = *reinterpret_cast<const int32x4*>(&cap[(8192 + ((k >> 1) & 3) * 512 + (lane >> 5) * 64 + q4 * 16) / 4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) dsv[4 * q4 + e] = __int_as_float(d4[e]);
                    }
                }
                const int2 ad = *reinterpret_cast<const int2*>(&cap[(12288 + (k & 7) * 256 + (lane & 31) * 8) / 4]);
                dal = __int_as_float(ad.x);
                c0l = __int_as_float(ad.y);
                __builtin_amdgcn_sched_barrier(0);
                F[(k + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bn, magic, 0, 0, 0);
            } else if constexpr (MODE == 4) {
                F[k & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, magic, 0, 0, 0);
            } else if constexpr (MODE != 1) {
                F[(k + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, magic, 0, 0, 0);
                if constexpr (MODE == 0 || MODE == 3) asm volatile("" : : "v"(F[(k + 1) & 1]));
            }
            if constexpr (MODE != 0) {
                int32x16 Fk;
                if constexpr (MODE == 2 || MODE >= 4) {
                    Fk = F[k & 1];
                } else {
                    asm volatile("" : "+v"(opaque));       // a new, unknown value every step
                    Fk = opaque;
                }
                if constexpr (MODE == 7) {
                    // the fold in groups of four: four independent first FMAs, then the four
                    // accumulating ones (no FMA waits on the one just before it)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float e[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) e[j] = fmaf(__int_as_float(Fk[4 * g + j]), dal, c0l);
                        asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
#pragma unroll
                        for (int j = 0; j < 4; ++j) y[k & 1][4 * g + j] = fmaf(e[j], dsv[4 * g + j], y[k & 1][4 * g + j]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = fmaf(__int_as_float(Fk[r]), dal, c0l);
                        y[k & 1][r] = fmaf(e, dsv[r], y[k & 1][r]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        a[0] += 1;
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += y[0][r] + y[1][r];
    __syncthreads();
    const int si = __float_as_int(s) ^ F[0][lane & 15] ^ F[1][3] ^ cap[(tx * 7) & 255];
    if (tx == 0) {
        out[4 * blockIdx.x + 0] = t1 - t0;
        out[4 * blockIdx.x + 1] = r1 - r0;
        out[4 * blockIdx.x + 2] = (uint64_t)(uint32_t)si;
        out[4 * blockIdx.x + 3] = 0;
    }
}

int check_device(int* cus)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -4;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return -4;
    const char* n = p.gcnArchName;
    if (!(n[0] == 'g' && n[1] == 'f' && n[2] == 'x' && n[3] == '9' && n[4] == '5' && n[5] == '0' &&
          (n[6] == 0 || n[6] == ':')))
        return -4;
    *cus = p.multiProcessorCount;
    return 0;
}

template <int MODE>
hipError_t launch_mode(int w, unsigned blocks, int iters, uint64_t* out, hipStream_t s)
{
    switch (w) {
    case 1: hipLaunchKernelGGL((step_kernel<MODE, 1>), dim3(blocks), dim3(256), 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL((step_kernel<MODE, 2>), dim3(blocks), dim3(256), 0, s, iters, out); break;
    case 3: hipLaunchKernelGGL((step_kernel<MODE, 3>), dim3(blocks), dim3(256), 0, s, iters, out); break;
    default: hipLaunchKernelGGL((step_kernel<MODE, 4>), dim3(blocks), dim3(256), 0, s, iters, out); break;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" int64_t qpg_calib_step_blocks(int waves_per_simd)
{
    int cus = 0;
    if (waves_per_simd < 1 || waves_per_simd > 4 || check_device(&cus) != 0) return 0;
    return (int64_t)cus * waves_per_simd;
}

extern "C" int qpg_calib_step(int mode, int waves_per_simd, int64_t iters, uint64_t* out, void* stream)
{
    if (!out || mode < 0 || mode > 7 || waves_per_simd < 1 || waves_per_simd > 4 || iters < 1 || iters > 10000000)
        return -1;
    if (((uintptr_t)out & 7) != 0) return -2;
    int cus = 0;
    const int dv = check_device(&cus);
    if (dv != 0) return dv;
    const unsigned blocks = (unsigned)(cus * waves_per_simd);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    switch (mode) {
    case 0: e = launch_mode<0>(waves_per_simd, blocks, (int)iters, out, s); break;
    case 1: e = launch_mode<1>(waves_per_simd, blocks, (int)iters, out, s); break;
    case 2: e = launch_mode<2>(waves_per_simd, blocks, (int)iters, out, s); break;
    case 3: e = launch_mode<3>(waves_per_simd, blocks, (int)iters, out, s); break;
    case 4: e = launch_mode<4>(waves_per_simd, blocks, (int)iters, out, s); break;
    case 5: e = launch_mode<5>(waves_per_simd, blocks, (int)iters, out, s); break;
    case 6: e = launch_mode<6>(waves_per_simd, blocks, (int)iters, out, s); break;
    default: e = launch_mode<7>(waves_per_simd, blocks, (int)iters, out, s); break;
    }
    return e == hipSuccess ? 0 : -3;
}
