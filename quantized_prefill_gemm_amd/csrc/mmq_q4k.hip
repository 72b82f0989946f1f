// q4_K x q8_1 MMQ kernel for gfx950 (MI355X).
//
// Y[i][j] = sum over 32-wide chunks c of
//           da_ic * dsv_jc * I_ijc  +  da_ic * ssum_ic * dmv_jc,
//   I_ijc = sum_{k in c} nib_jk * q_ik (exact int32),  dsv = d*sc,  dmv = -dmin*m
// -- the two-term fold of "r28 - Direction-A raw-nibble NB kernel", sec. 2.3, with the
// raw-nibble B operand of the same page (sec. 3.2): low nibble for even sub-blocks, high
// nibble for odd ones, no sign extension, the unsigned 0..15 value fed to the integer
// product as is.
//
// MI355X design (not the pages' GB10 one):
//  * Workgroup tile 64 tokens x 128 weight rows, 4 waves; wave w owns weight rows
//    32w..32w+31 of the tile and all 64 tokens (two 32x32 output sub-tiles).
//  * Per super-block (256 k) the workgroup stages, with 16-byte coalesced global loads,
//    the raw q4_K qs bytes (128 B per row) and the q8_1 int8 tile into LDS, and decodes
//    the block headers once into per-(row, sub-block) f32 terms.
//  * Integer stage: one v_mfma_i32_32x32x32_i8 per (32x32 sub-tile, chunk). K = 32 is
//    exactly one q8_1 block and one q4_K sub-block, so no two scales ever share an
//    integer accumulator. A 16-byte LDS read of raw qs serves two chunks: the low
//    nibbles (& 0x0F0F0F0F) are chunk 2p, the high nibbles (>> 4 & 0x0F0F0F0F) chunk 2p+1.
//  * The MFMA accumulates onto the bits of 1.5*2^23, so its int32 result read as f32 is
//    1.5*2^23 + I exactly (|I| <= 15*127*32 < 2^22). One FMA with the per-row constant
//    c0 = -1.5*2^23*dsv gives round(dsv*I) (dsv has <= 17 significant bits, so c0 is
//    exact), and a second FMA with da accumulates: two VALU ops per output per chunk.
//  * Min term: per super-block, sum_s (da*ssum)_is * m_js is a K=8 product. da*ssum is an
//    exact f32 (11 + 12 bits); it is split into three bf16 pieces whose sum is exact,
//    m (0..63) is exact in bf16, and two v_mfma_f32_32x32x16_bf16 form the product with
//    f32 accumulation; one FMA with -dmin per super-block folds it into Y.
//  * The "isums" instantiation runs the same staging, unpack and MFMA code and stores the
//    integer sums instead of folding them (the bit-exact witness of the integer stage).
#include "qpg_common.h"

namespace qpg {
namespace q4k {

typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64;            // tokens per workgroup tile
constexpr int TN = 128;           // weight rows per workgroup tile
constexpr int AQ_STRIDE = 272;    // LDS bytes per token row of the q tile (256 + 16 pad)
constexpr int BQ_STRIDE = 144;    // LDS bytes per weight row of the qs tile (128 + 16 pad)
constexpr int BS_STRIDE = 80;     // per weight row: dsv[8] f32, c0[8] f32, m[8] bf16
constexpr int AX_STRIDE = 48;     // per token: x1[8], x2[8], x3[8] bf16 pieces of da*ssum

// Strides are chosen so that 16 lanes reading 16 bytes each at consecutive rows hit 16
// distinct 16-byte bank groups of the 64-bank LDS (stride mod 256 is an odd multiple of
// 16 or 48/80/144-type values whose multiples are distinct mod 256).
struct alignas(16) Smem {
    alignas(16) uint8_t aq[TM * AQ_STRIDE];          // q8_1 int8 tile of the super-block
    alignas(16) float ada[8][2][2][16];              // da in C-register order: [chunk][subtile][k-group][r]
    alignas(16) uint8_t ax[TM * AX_STRIDE];          // min-term A operand pieces
    alignas(16) uint8_t bq[TN * BQ_STRIDE];          // raw qs bytes of the super-block
    alignas(16) uint8_t bs[TN * BS_STRIDE];          // decoded per-(row, sub-block) scale terms
    alignas(16) float bnd[TN];                       // -dmin per row
};

__device__ __forceinline__ void tile_coords(int& m_tile, int& n_tile, int tiles_m, int total)
{
    // Workgroups are dispatched round-robin over the 8 XCDs (bid % 8). Give each XCD a
    // contiguous range of tiles, M fastest, so the workgroups sharing a weight tile run
    // on one XCD and read it into that XCD's L2 once.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, k = bid >> 3;
    const int q = total >> 3, r = total & 7;
    const int t = xcd * q + (xcd < r ? xcd : r) + k;
    m_tile = t % tiles_m;
    n_tile = t / tiles_m;
}

template <bool ISUMS>
__global__ void __launch_bounds__(256) mmq_q4K_kernel(const uint8_t* __restrict__ W,
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
    const int nsb = K / QK_K, nc = K / QK8;
    const size_t wrow = (size_t)nsb * Q4K_BYTES;
    const int jl = 32 * wave + l32;      // this lane's weight row within the tile

    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_BITS;
    floatx16 y[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[a][r] = 0.0f;

    for (int sb = 0; sb < nsb; ++sb) {
        // ---------------- stage A: q8 tile (64 tokens x 256 B), 16-byte granules
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int g = it * 256 + tid, t = g >> 4, part = g & 15;
            int32x4 v = {0, 0, 0, 0};
            if (m0 + t < M)
                v = *reinterpret_cast<const int32x4*>(qplane + (size_t)(m0 + t) * K + sb * QK_K + part * 16);
            *reinterpret_cast<int32x4*>(sm.aq + t * AQ_STRIDE + part * 16) = v;
        }
        // ---------------- stage A: headers -> da (C order) and bf16 pieces of da*ssum
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int h = it * 256 + tid, t = h >> 3, c = h & 7;
            uint32_t hw = 0;
            if (m0 + t < M) hw = hdr[(size_t)(m0 + t) * nc + sb * 8 + c];
            const float da = half_bits_to_float(hw & 0xFFFFu);
            const float xs = da * (float)(int16_t)(hw >> 16);            // exact
            const int a = t >> 5, tt = t & 31;
            sm.ada[c][a][(tt >> 2) & 1][4 * (tt >> 3) + (tt & 3)] = da;
            const uint32_t b1 = f32_to_bf16_bits(xs);
            const float r1 = xs - bf16_bits_to_f32(b1);                    // exact
            const uint32_t b2 = f32_to_bf16_bits(r1);
            const float r2 = r1 - bf16_bits_to_f32(b2);                    // exact
            const uint32_t b3 = f32_to_bf16_bits(r2);                      // r2 has <= 8 bits
            uint16_t* ax = reinterpret_cast<uint16_t*>(sm.ax + t * AX_STRIDE);
            ax[c] = (uint16_t)b1;
            ax[8 + c] = (uint16_t)b2;
            ax[16 + c] = (uint16_t)b3;
        }
        // ---------------- stage B: raw qs (128 rows x 128 B)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int g = it * 256 + tid, j = g >> 3, part = g & 7;
            int32x4 v = {0, 0, 0, 0};
            if (n0 + j < N)
                v = *reinterpret_cast<const int32x4*>(W + (size_t)(n0 + j) * wrow + (size_t)sb * Q4K_BYTES + 16 +
                                                      part * 16);
            *reinterpret_cast<int32x4*>(sm.bq + j * BQ_STRIDE + part * 16) = v;
        }
        // ---------------- stage B: decode d, dmin and the eight 6-bit (sc, m) pairs
        if (tid < TN) {
            const int j = tid;
            uint32x4 hv = {0u, 0u, 0u, 0u};
            if (n0 + j < N)
                hv = *reinterpret_cast<const uint32x4*>(W + (size_t)(n0 + j) * wrow + (size_t)sb * Q4K_BYTES);
            const float d = half_bits_to_float(hv[0] & 0xFFFFu);
            const float dmin = half_bits_to_float(hv[0] >> 16);
            const uint32_t S0 = hv[1], S1 = hv[2], S2 = hv[3];   // packed bytes 0-3, 4-7, 8-11
            float* bs = reinterpret_cast<float*>(sm.bs + j * BS_STRIDE);
            uint16_t* bm = reinterpret_cast<uint16_t*>(sm.bs + j * BS_STRIDE + 64);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                uint32_t sc, m;
                if (s < 4) {
                    sc = (S0 >> (8 * s)) & 63u;
                    m = (S1 >> (8 * s)) & 63u;
                } else {
                    const int s4 = 8 * (s - 4);
                    sc = ((S2 >> s4) & 15u) | (((S0 >> s4) >> 6 & 3u) << 4);
                    m = ((S2 >> s4) >> 4 & 15u) | (((S1 >> s4) >> 6 & 3u) << 4);
                }
                const float dsv = d * (float)sc;                           // exact (17 bits)
                bs[s] = dsv;
                bs[8 + s] = -MAGIC_F * dsv;                                 // exact
                bm[s] = (uint16_t)(__float_as_uint((float)m) >> 16);       // m exact in bf16
            }
            sm.bnd[j] = -dmin;
        }
        __syncthreads();

        // ---------------- compute: 8 chunks x 2 sub-tiles, then the min term
        const floatx4* bsp = reinterpret_cast<const floatx4*>(sm.bs + jl * BS_STRIDE);
        const floatx4 dsv_lo = bsp[0], dsv_hi = bsp[1], c0_lo = bsp[2], c0_hi = bsp[3];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32x4 raw = *reinterpret_cast<const uint32x4*>(sm.bq + jl * BQ_STRIDE + 32 * p + 16 * hg);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int c = 2 * p + half;
                const uint32x4 bu = half ? ((raw >> 4u) & 0x0F0F0F0Fu) : (raw & 0x0F0F0F0Fu);
                int32x4 b;
                __builtin_memcpy(&b, &bu, 16);
                const float dsv = c < 4 ? dsv_lo[c & 3] : dsv_hi[c & 3];
                const float c0 = c < 4 ? c0_lo[c & 3] : c0_hi[c & 3];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const int32x4 av =
                        *reinterpret_cast<const int32x4*>(sm.aq + (32 * a + l32) * AQ_STRIDE + 32 * c + 16 * hg);
                    const int32x16 F = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b, magic, 0, 0, 0);
                    if constexpr (ISUMS) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = m0 + 32 * a + c_row(r, lane), col = n0 + jl;
                            if (row < M && col < N)
                                S[((size_t)row * N + col) * nc + sb * 8 + c] = F[r] - MAGIC_BITS;
                        }
                    } else {
                        const floatx4* dap = reinterpret_cast<const floatx4*>(&sm.ada[c][a][hg][0]);
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const floatx4 da = dap[q4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int r = 4 * q4 + e;
                                const float ev = fmaf(__int_as_float(F[r]), dsv, c0);   // dsv * I
                                y[a][r] = fmaf(ev, da[e], y[a][r]);
                            }
                        }
                    }
                }
            }
        }
        if constexpr (!ISUMS) {
            bf16x8 mB, mB2;
            const int32x4 mraw = *reinterpret_cast<const int32x4*>(sm.bs + jl * BS_STRIDE + 64);
            const int32x4 zero4 = {0, 0, 0, 0};
            const int32x4 mraw2 = hg ? zero4 : mraw;
            __builtin_memcpy(&mB, &mraw, 16);
            __builtin_memcpy(&mB2, &mraw2, 16);
            const float nd = sm.bnd[jl];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                bf16x8 x12, x3;
                __builtin_memcpy(&x12, sm.ax + (32 * a + l32) * AX_STRIDE + 16 * hg, 16);
                __builtin_memcpy(&x3, sm.ax + (32 * a + l32) * AX_STRIDE + 32, 16);
                floatx16 R;
#pragma unroll
                for (int r = 0; r < 16; ++r) R[r] = 0.0f;
                // k-group 0 carries x1, k-group 1 carries x2 (against m in both groups);
                // then x3 against m in group 0 only.
                R = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x12, mB, R, 0, 0, 0);
                R = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x3, mB2, R, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) y[a][r] = fmaf(R[r], nd, y[a][r]);
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

}  // namespace q4k
}  // namespace qpg

hipError_t qpg_launch_mmq_q4K(const void* w, const void* xq, float* y, int32_t* isums, int64_t M, int64_t N,
                              int64_t K, hipStream_t s)
{
    using namespace qpg::q4k;
    const int tiles_m = (int)((M + TM - 1) / TM);
    const int tiles_n = (int)((N + TN - 1) / TN);
    const int total = tiles_m * tiles_n;
    const int8_t* qplane = static_cast<const int8_t*>(xq);
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(qplane + M * K);
    if (isums)
        hipLaunchKernelGGL(mmq_q4K_kernel<true>, dim3(total), dim3(256), 0, s, static_cast<const uint8_t*>(w),
                           qplane, hdr, y, isums, (int)M, (int)N, (int)K, tiles_m, total);
    else
        hipLaunchKernelGGL(mmq_q4K_kernel<false>, dim3(total), dim3(256), 0, s, static_cast<const uint8_t*>(w),
                           qplane, hdr, y, isums, (int)M, (int)N, (int)K, tiles_m, total);
    return hipGetLastError();
}
