// q6_K x q8_1 MMQ kernel for gfx950 (MI355X).
//
// Y[i][j] = sum over 16-wide sub-blocks u of da_{i,u/2} * (d*sc)_{ju} * J_iju,
//   J_iju = sum_{k in u} (q6_jk - 32) * q_ik  (exact int32).
// q6_K carries one int8 scale per 16 weights, so each 32-wide q8_1 chunk holds two
// integer products with different scales -- the "KSPLIT=2" structure of the q6_K kernel
// of "r40 - __launch_bounds__(256,3) third resident block" (sec. 5): two 16-k products
// per chunk.
//
// MI355X design:
//  * Same tile as the q4_K kernel (64 tokens x 128 weight rows, 4 waves, each wave 32
//    weight rows x 64 tokens = two 32x32 sub-tiles).
//  * Integer stage: v_mfma_i32_32x32x16_i8 per (sub-tile, 16-wide sub-block). The B
//    operand is the unsigned 6-bit value q6 = low4 | high2 << 4 (0..63, a valid int8);
//    the "- 32" is applied by the matrix core itself: a first MFMA multiplies the
//    activations by a constant -32 operand onto the bits of 1.5*2^23, the second adds
//    q6 * q onto that, so the int32 result read as f32 is 1.5*2^23 + J exactly
//    (|J| <= 32*127*16 < 2^22) with no per-byte VALU work for the offset.
//  * Fold: e = fma(F, d*sc, -1.5*2^23*d*sc) = round(d*sc*J); y = fma(e, da, y).
//  * q6_K rows start only 2-byte aligned (210-byte blocks), so the staging reads aligned
//    dwords and shifts them into place with v_alignbyte (no misaligned wide loads).
//  * LDS layout: inside every 32-byte group of q, ql and qh, the 8-byte pieces 1 and 2
//    are swapped at staging, so one 16-byte LDS read gives a lane its 8 bytes of both
//    16-wide sub-blocks of a chunk (k-group l>>5 of each K=16 MFMA).
#include "qpg_common.h"

namespace qpg {
namespace q6k {

typedef unsigned uint32x2 __attribute__((ext_vector_type(2)));
typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64;
constexpr int TN = 128;
constexpr int AQ_STRIDE = 272;    // q tile row (256 + 16 pad)
constexpr int BL_STRIDE = 144;    // ql row (128 + 16 pad)
constexpr int BH_STRIDE = 80;     // qh row (64 + 16 pad)
constexpr int BS_STRIDE = 80;     // d*sc[16] f32 (64 + 16 pad)

struct alignas(16) Smem {
    alignas(16) uint8_t aq[TM * AQ_STRIDE];
    alignas(16) float ada[8][2][2][16];
    alignas(16) uint8_t bl[TN * BL_STRIDE];
    alignas(16) uint8_t bh[TN * BH_STRIDE];
    alignas(16) uint8_t bs[TN * BS_STRIDE];
};

__device__ __forceinline__ void tile_coords(int& m_tile, int& n_tile, int tiles_m, int total)
{
    const int bid = blockIdx.x;
    const int xcd = bid & 7, k = bid >> 3;
    const int q = total >> 3, r = total & 7;
    const int t = xcd * q + (xcd < r ? xcd : r) + k;
    m_tile = t % tiles_m;
    n_tile = t / tiles_m;
}

__device__ __forceinline__ uint32_t ld32(const uint8_t* p)
{
    return *reinterpret_cast<const uint32_t*>(p);     // p is 4-byte aligned
}

// 16 bytes starting at the 2-byte aligned address base + off, read as aligned dwords
// from [base + off - sh, base + off - sh + 16 + 4*(sh != 0)).
__device__ __forceinline__ uint32x4 ld16_a2(const uint8_t* p, uint32_t sh)
{
    const uint8_t* a = p - sh;
    uint32x4 v;
    const uint32_t w0 = ld32(a), w1 = ld32(a + 4), w2 = ld32(a + 8), w3 = ld32(a + 12);
    if (sh) {
        const uint32_t w4 = ld32(a + 16);
        v[0] = __builtin_amdgcn_alignbyte(w1, w0, 2);
        v[1] = __builtin_amdgcn_alignbyte(w2, w1, 2);
        v[2] = __builtin_amdgcn_alignbyte(w3, w2, 2);
        v[3] = __builtin_amdgcn_alignbyte(w4, w3, 2);
    } else {
        v[0] = w0; v[1] = w1; v[2] = w2; v[3] = w3;
    }
    return v;
}

// Store a 16-byte granule that sits at byte 16*gi (gi = 0/1) of a 32-byte group into the
// permuted group: bytes 0-7 go to 8*gi, bytes 8-15 to 16 + 8*gi.
__device__ __forceinline__ void st_perm(uint8_t* group, int gi, uint32x4 v)
{
    uint32x2 lo = {v[0], v[1]}, hi = {v[2], v[3]};
    *reinterpret_cast<uint32x2*>(group + 8 * gi) = lo;
    *reinterpret_cast<uint32x2*>(group + 16 + 8 * gi) = hi;
}

template <bool ISUMS>
__global__ void __launch_bounds__(256) mmq_q6K_kernel(const uint8_t* __restrict__ W,
                                                      const int8_t* __restrict__ qplane,
                                                      const uint32_t* __restrict__ hdr,
                                                      float* __restrict__ Y,
                                                      int32_t* __restrict__ S,
                                                      int M, int N, int K, int tiles_m, int total)
{
    __shared__ Smem sm;
    int m_tile, n_tile;
    tile_coords(m_tile, n_tile, tiles_m, total);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hg = lane >> 5, l32 = lane & 31;
    const int m0 = m_tile * TM, n0 = n_tile * TN;
    const int nsb = K / QK_K, nc = K / QK8, nu = K / 16;
    const size_t wrow = (size_t)nsb * Q6K_BYTES;
    const int jl = 32 * wave + l32;

    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_BITS;
    const long minus32 = (long)0xE0E0E0E0E0E0E0E0ull;     // eight int8 -32
    floatx16 y[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[a][r] = 0.0f;

    for (int sb = 0; sb < nsb; ++sb) {
        // ---------------- stage A: q8 tile, 16-byte granule p of a row is sub-block p
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int g = it * 256 + tid, t = g >> 4, part = g & 15;
            uint32x4 v = {0u, 0u, 0u, 0u};
            if (m0 + t < M)
                v = *reinterpret_cast<const uint32x4*>(qplane + (size_t)(m0 + t) * K + sb * QK_K + part * 16);
            st_perm(sm.aq + t * AQ_STRIDE + 32 * (part >> 1), part & 1, v);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int h = it * 256 + tid, t = h >> 3, c = h & 7;
            uint32_t hw = 0;
            if (m0 + t < M) hw = hdr[(size_t)(m0 + t) * nc + sb * 8 + c];
            const int a = t >> 5, tt = t & 31;
            sm.ada[c][a][(tt >> 2) & 1][4 * (tt >> 3) + (tt & 3)] = half_bits_to_float(hw & 0xFFFFu);
        }
        // ---------------- stage B: ql (8 granules) and qh (4 granules) per row
#pragma unroll
        for (int it = 0; it < 6; ++it) {
            const int g = it * 256 + tid, j = g / 12, gi = g - 12 * j;
            uint32x4 v = {0u, 0u, 0u, 0u};
            if (n0 + j < N) {
                const size_t off = (size_t)(n0 + j) * wrow + (size_t)sb * Q6K_BYTES;
                v = ld16_a2(W + off + 16 * gi, (uint32_t)(off & 2));
            }
            if (gi < 8)
                st_perm(sm.bl + j * BL_STRIDE + 32 * (gi >> 1), gi & 1, v);
            else
                st_perm(sm.bh + j * BH_STRIDE + 32 * ((gi - 8) >> 1), gi & 1, v);
        }
        // ---------------- stage B: d * sc[u] per row
        if (tid < TN) {
            const int j = tid;
            float* bs = reinterpret_cast<float*>(sm.bs + j * BS_STRIDE);
            if (n0 + j < N) {
                const size_t off = (size_t)(n0 + j) * wrow + (size_t)sb * Q6K_BYTES;
                const uint32_t sh = (uint32_t)(off & 2);
                const uint32x4 scw = ld16_a2(W + off + 192, sh);
                const uint32_t dbits = *reinterpret_cast<const uint16_t*>(W + off + 208);
                const float d = half_bits_to_float(dbits);
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int sc = (int)(int8_t)(scw[u >> 2] >> (8 * (u & 3)));
                    bs[u] = d * (float)sc;                          // exact (19 bits)
                }
            } else {
#pragma unroll
                for (int u = 0; u < 16; ++u) bs[u] = 0.0f;
            }
        }
        __syncthreads();

        // ---------------- compute
        const floatx4* bsp = reinterpret_cast<const floatx4*>(sm.bs + jl * BS_STRIDE);
        floatx4 dsc4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dsc4[i] = bsp[i];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const int h = cc >> 2, g = cc & 3;
            const uint32x4 ql = *reinterpret_cast<const uint32x4*>(sm.bl + jl * BL_STRIDE + 64 * h + 32 * (g & 1) + 16 * hg);
            const uint32x4 qh = *reinterpret_cast<const uint32x4*>(sm.bh + jl * BH_STRIDE + 32 * h + 16 * hg);
            uint32x4 q6;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = (ql[e] >> (4 * (g >> 1))) & 0x0F0F0F0Fu;
                const uint32_t hi = ((qh[e] >> (2 * g)) & 0x03030303u) << 4;
                q6[e] = lo | hi;
            }
            const long b0 = (long)(((unsigned long)q6[1] << 32) | q6[0]);
            const long b1 = (long)(((unsigned long)q6[3] << 32) | q6[2]);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const uint32x4 av =
                    *reinterpret_cast<const uint32x4*>(sm.aq + (32 * a + l32) * AQ_STRIDE + 32 * cc + 16 * hg);
                const long a0 = (long)(((unsigned long)av[1] << 32) | av[0]);
                const long a1 = (long)(((unsigned long)av[3] << 32) | av[2]);
                int32x16 F0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a0, minus32, magic, 0, 0, 0);
                F0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a0, b0, F0, 0, 0, 0);
                int32x16 F1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a1, minus32, magic, 0, 0, 0);
                F1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a1, b1, F1, 0, 0, 0);
                if constexpr (ISUMS) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m0 + 32 * a + c_row(r, lane), col = n0 + jl;
                        if (row < M && col < N) {
                            int32_t* dst = S + ((size_t)row * N + col) * nu + sb * 16 + 2 * cc;
                            dst[0] = F0[r] - MAGIC_BITS;
                            dst[1] = F1[r] - MAGIC_BITS;
                        }
                    }
                } else {
                    const float s0 = dsc4[(2 * cc) >> 2][(2 * cc) & 3];
                    const float s1 = dsc4[(2 * cc + 1) >> 2][(2 * cc + 1) & 3];
                    const float c00 = -MAGIC_F * s0, c01 = -MAGIC_F * s1;
                    const floatx4* dap = reinterpret_cast<const floatx4*>(&sm.ada[cc][a][hg][0]);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const floatx4 da = dap[q4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * q4 + e;
                            const float e0 = fmaf(__int_as_float(F0[r]), s0, c00);
                            const float e1 = fmaf(__int_as_float(F1[r]), s1, c01);
                            y[a][r] = fmaf(e0 + e1, da[e], y[a][r]);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!ISUMS) {
        const int col = n0 + jl;
        if (col < N) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + 32 * a + c_row(r, lane);
                    if (row < M) Y[(size_t)row * N + col] = y[a][r];
                }
        }
    }
}

}  // namespace q6k
}  // namespace qpg

hipError_t qpg_launch_mmq_q6K(const void* w, const void* xq, float* y, int32_t* isums, int64_t M, int64_t N,
                              int64_t K, hipStream_t s)
{
    using namespace qpg::q6k;
    const int tiles_m = (int)((M + TM - 1) / TM);
    const int tiles_n = (int)((N + TN - 1) / TN);
    const int total = tiles_m * tiles_n;
    const int8_t* qplane = static_cast<const int8_t*>(xq);
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(qplane + M * K);
    if (isums)
        hipLaunchKernelGGL(mmq_q6K_kernel<true>, dim3(total), dim3(256), 0, s, static_cast<const uint8_t*>(w),
                           qplane, hdr, y, isums, (int)M, (int)N, (int)K, tiles_m, total);
    else
        hipLaunchKernelGGL(mmq_q6K_kernel<false>, dim3(total), dim3(256), 0, s, static_cast<const uint8_t*>(w),
                           qplane, hdr, y, isums, (int)M, (int)N, (int)K, tiles_m, total);
    return hipGetLastError();
}
