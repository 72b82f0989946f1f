// q6_K x q8_1 MMQ kernel for gfx950 (MI355X).
//
// Y[i][j] = sum over 16-wide sub-blocks u of da_{i,u/2} * (d*sc)_{ju} * J_iju,
//   J_iju = sum_{k in u} (q6_jk - 32) * q_ik  (exact int32).
// q6_K carries one int8 scale per 16 weights, so each 32-wide q8_1 chunk holds two
// integer products with different scales -- the two 16-k products per 32-k chunk of the
// q6_K kernel of "r40 - __launch_bounds__(256,3) third resident block" (sec. 5).
//
// MI355X design:
//  * Tile 64 tokens x 128 weight rows, 4 waves; wave w = weight rows 32w..32w+31 (MFMA row
//    side) x 64 tokens (two 32x32 sub-tiles on the column side): da is one value per lane,
//    d*sc is read once per sub-block for both token sub-tiles.
//  * Integer stage: v_mfma_i32_32x32x16_i8 per (token sub-tile, 16-wide sub-block). The
//    weight operand v = q6 - 32 is assembled per byte in registers from the raw ql / qh bytes
//    in LDS: q6 = low4 | high2 << 4, and v = ((q6 | 0x80) - 0x20) ^ 0x80 turns the unsigned
//    6-bit value into the signed int8 q6 - 32 without any borrow between bytes.
//  * The MFMA accumulates onto the bits of 1.5*2^23, so its int32 result read as f32 is
//    1.5*2^23 + J exactly (|J| <= 32*127*16 < 2^22): e = fma(F, da, -1.5*2^23*da) is
//    round(da*J) and y = fma(e, d*sc, y). Two VALU ops per output and sub-block.
//  * q6_K rows start only 2-byte aligned (210-byte blocks): staging reads aligned dwords and
//    shifts them into place with v_alignbyte, never a misaligned wide load.
//  * LDS: inside every 32-byte group of q, ql and qh the 8-byte pieces 1 and 2 are swapped at
//    staging, so one 16-byte read gives a lane its 8 bytes of both sub-blocks of a chunk
//    (k-group l>>5 of each K=16 MFMA). Rows are XOR-swizzled in 16-byte granules so reads of
//    16 consecutive rows hit 16 distinct bank groups.
#include "qpg_common.h"

namespace qpg {
namespace q6k {

typedef unsigned uint32x2 __attribute__((ext_vector_type(2)));
typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64;
constexpr int TN = 128;
constexpr int DA_STRIDE = 20;     // floats per token: per chunk pair p: da_2p, da_2p+1, c0_2p, c0_2p+1 (+pad)

struct alignas(16) Smem {
    alignas(16) uint8_t aq[TM * 256];          // q8 tile, permuted pieces, granule g of token t at g ^ (t & 15)
    alignas(16) uint8_t bl[TN * 128];          // ql, permuted pieces, granule g of row j at g ^ ((j >> 1) & 7)
    alignas(16) uint8_t bh[TN * 64];           // qh, permuted pieces, granule g of row j at g ^ ((j >> 2) & 3)
    alignas(16) float bdsc[16][TN];            // d*sc per sub-block, rows in C-register order per wave
    alignas(16) float ada[TM * DA_STRIDE];     // da and -1.5*2^23*da per token and chunk
};

__device__ __forceinline__ void tile_coords(int& m_tile, int& n_tile, int tiles_m, int total)
{
    // round-robin XCD dispatch: give each XCD a contiguous range of tiles, M fastest, so
    // the workgroups sharing a weight tile run on one XCD (one L2)
    const int bid = blockIdx.x;
    const int xcd = bid & 7, k = bid >> 3;
    const int q = total >> 3, r = total & 7;
    const int t = xcd * q + (xcd < r ? xcd : r) + k;
    m_tile = t % tiles_m;
    n_tile = t / tiles_m;
}

__device__ __forceinline__ int c_pos(int jj) { return 16 * ((jj >> 2) & 1) + 4 * (jj >> 3) + (jj & 3); }

__device__ __forceinline__ uint32_t ld32(const uint8_t* p)
{
    return *reinterpret_cast<const uint32_t*>(p);     // p is 4-byte aligned
}

// 16 bytes starting at the 2-byte aligned address p, read as aligned dwords from
// [p - sh, p - sh + 16 + 4*(sh != 0)), sh = p & 2.
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

// A 16-byte granule at byte 16*gi (gi = 0/1) of a 32-byte group, stored with the group's
// pieces 1 and 2 swapped: bytes 0-7 go to piece gi, bytes 8-15 to piece 2 + gi. `grp` is the
// group's LDS base; the pieces land in granules (2*G + 0/1) ^ sw of the row.
__device__ __forceinline__ void st_perm(uint8_t* row, int G, int gi, int sw, uint32x4 v)
{
    const uint32x2 lo = {v[0], v[1]}, hi = {v[2], v[3]};
    // piece P (0..3) of group G sits in granule 2G + (P >> 1), half (P & 1)
    *reinterpret_cast<uint32x2*>(row + 16 * ((2 * G + 0) ^ sw) + 8 * gi) = lo;   // piece gi
    *reinterpret_cast<uint32x2*>(row + 16 * ((2 * G + 1) ^ sw) + 8 * gi) = hi;   // piece 2 + gi
}

template <bool ISUMS>
__global__ void __launch_bounds__(256, ISUMS ? 1 : 2) mmq_q6K_kernel(const uint8_t* __restrict__ W,
                                                                     const int8_t* __restrict__ qplane,
                                                                     const uint32_t* __restrict__ hdr,
                                                                     float* __restrict__ Y,
                                                                     int32_t* __restrict__ S,
                                                                     int M, int N, int K, int tiles_m, int total)
{
    __shared__ Smem sm;
    int m_tile, n_tile;
    tile_coords(m_tile, n_tile, tiles_m, total);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = lane >> 5, l32 = lane & 31;
    const int m0 = m_tile * TM, n0 = n_tile * TN;
    const int nsb = K / QK_K, nc = K / QK8, nu = K / 16;
    const size_t wrow = (size_t)nsb * Q6K_BYTES;

    const int rows_t = min(TM, M - m0);
    const __amdgpu_buffer_rsrc_t rQ =
        __builtin_amdgcn_make_buffer_rsrc((void*)(qplane + (size_t)m0 * K), 0, rows_t * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rH =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hdr + (size_t)m0 * nc), 0, rows_t * nc * 4, 0x00020000);

    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_BITS;
    floatx16 y[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[a][r] = 0.0f;

    const int wr = 32 * wave + l32;                  // weight row of this lane's A operand
    int tk[2];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) tk[ts] = 32 * ts + l32;

    for (int sb = 0; sb < nsb; ++sb) {
        // ---------------- stage A: q8 tile; 16-byte granule p of a row is sub-block p
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int g = it * 256 + tid, t = g >> 4, part = g & 15;
            const uint32x4 v = __builtin_bit_cast(
                uint32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, t * K + sb * QK_K + part * 16, 0, 0));
            st_perm(sm.aq + t * 256, part >> 1, part & 1, t & 15, v);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int h = it * 256 + tid, t = h >> 3, c = h & 7;
            const uint32_t hw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rH, (t * nc + sb * 8 + c) * 4, 0, 0);
            const float da = half_bits_to_float(hw & 0xFFFFu);
            float* ad = sm.ada + t * DA_STRIDE + 4 * (c >> 1) + (c & 1);
            ad[0] = da;
            ad[2] = -MAGIC_F * da;                                                  // exact
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
                st_perm(sm.bl + j * 128, gi >> 1, gi & 1, (j >> 1) & 7, v);
            else
                st_perm(sm.bh + j * 64, (gi - 8) >> 1, gi & 1, (j >> 2) & 3, v);
        }
        // ---------------- stage B: d * sc[u] per row, in C-register order
        if (tid < TN) {
            const int j = tid;
            const int pos = 32 * (j >> 5) + c_pos(j & 31);
            if (n0 + j < N) {
                const size_t off = (size_t)(n0 + j) * wrow + (size_t)sb * Q6K_BYTES;
                const uint32x4 scw = ld16_a2(W + off + 192, (uint32_t)(off & 2));
                const float d = half_bits_to_float(*reinterpret_cast<const uint16_t*>(W + off + 208));
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    sm.bdsc[u][pos] = d * (float)(int)(int8_t)(scw[u >> 2] >> (8 * (u & 3)));   // exact
            } else {
#pragma unroll
                for (int u = 0; u < 16; ++u) sm.bdsc[u][pos] = 0.0f;
            }
        }
        __syncthreads();

        // ---------------- integer stage + fold
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            // keep each chunk's loads and products together: bounds the live registers to one
            // chunk's operands. (Two resident workgroups per CU: at three the 168-register budget
            // spills, and the spilling form measured 1.6x slower.)
            __builtin_amdgcn_sched_barrier(0);
            const int h = cc >> 2, g = cc & 3;
            // weight operand for both sub-blocks of the chunk: 16 bytes of ql and of qh
            const uint32x4 ql = *reinterpret_cast<const uint32x4*>(
                sm.bl + wr * 128 + 16 * ((4 * h + 2 * (g & 1) + hg) ^ ((wr >> 1) & 7)));
            const uint32x4 qh = *reinterpret_cast<const uint32x4*>(
                sm.bh + wr * 64 + 16 * ((2 * h + hg) ^ ((wr >> 2) & 3)));
            uint32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = (ql[e] >> (4 * (g >> 1))) & 0x0F0F0F0Fu;
                const uint32_t hi = ((qh[e] >> (2 * g)) & 0x03030303u) << 4;
                const uint32_t q6 = lo | hi | 0x80808080u;                  // bit 7 set: no borrow below
                v[e] = (q6 - 0x20202020u) ^ 0x80808080u;                    // signed q6 - 32 per byte
            }
            const long a0 = (long)(((unsigned long)v[1] << 32) | v[0]);    // sub-block 2cc, k-group hg
            const long a1 = (long)(((unsigned long)v[3] << 32) | v[2]);    // sub-block 2cc+1
            floatx4 s0[4], s1[4];
            if constexpr (!ISUMS) {
                const floatx4* p0 = reinterpret_cast<const floatx4*>(&sm.bdsc[2 * cc][32 * wave + 16 * hg]);
                const floatx4* p1 = reinterpret_cast<const floatx4*>(&sm.bdsc[2 * cc + 1][32 * wave + 16 * hg]);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    s0[q4] = p0[q4];
                    s1[q4] = p1[q4];
                }
            }
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                const uint32x4 bq = *reinterpret_cast<const uint32x4*>(
                    sm.aq + tk[ts] * 256 + 16 * ((2 * cc + hg) ^ (tk[ts] & 15)));
                const long b0 = (long)(((unsigned long)bq[1] << 32) | bq[0]);
                const long b1 = (long)(((unsigned long)bq[3] << 32) | bq[2]);
                const int32x16 F0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a0, b0, magic, 0, 0, 0);
                const int32x16 F1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a1, b1, magic, 0, 0, 0);
                if constexpr (ISUMS) {
                    const int tok = m0 + tk[ts];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = n0 + 32 * wave + c_row(r, lane);
                        if (tok < M && row < N) {
                            int32_t* dst = S + ((size_t)tok * N + row) * nu + sb * 16 + 2 * cc;
                            dst[0] = F0[r] - MAGIC_BITS;
                            dst[1] = F1[r] - MAGIC_BITS;
                        }
                    }
                } else {
                    const floatx4 dc = *reinterpret_cast<const floatx4*>(sm.ada + tk[ts] * DA_STRIDE + 4 * (cc >> 1));
                    const float da = dc[cc & 1], c0 = dc[2 + (cc & 1)];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * q4 + e;
                            const float e0 = fmaf(__int_as_float(F0[r]), da, c0);    // round(da * J0)
                            const float e1 = fmaf(__int_as_float(F1[r]), da, c0);    // round(da * J1)
                            y[ts][r] = fmaf(e0, s0[q4][e], y[ts][r]);
                            y[ts][r] = fmaf(e1, s1[q4][e], y[ts][r]);
                        }
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!ISUMS) {
        // lane (ts, l32) holds token m0 + 32ts + l32; register group b = r>>2 holds the four
        // consecutive weight rows n0 + 32*wave + 8b + 4hg + 0..3
        const bool vec = ((N & 3) == 0) && ((((uintptr_t)Y) & 15) == 0);
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {
            const int tok = m0 + tk[ts];
            if (tok >= M) continue;
            float* yrow = Y + (size_t)tok * N;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int row = n0 + 32 * wave + 8 * b + 4 * hg;
                if (vec && row + 3 < N) {
                    floatx4 v = {y[ts][4 * b], y[ts][4 * b + 1], y[ts][4 * b + 2], y[ts][4 * b + 3]};
                    *reinterpret_cast<floatx4*>(yrow + row) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (row + e < N) yrow[row + e] = y[ts][4 * b + e];
                }
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
