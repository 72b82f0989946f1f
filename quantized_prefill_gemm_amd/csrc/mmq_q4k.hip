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
//    32w..32w+31 and all 64 tokens: two 32x32 output sub-tiles with the WEIGHT rows on
//    the MFMA row side and the tokens on the column side, so each lane's 16 accumulators
//    share one token: da is one register per lane, the per-row d*sc is read once per
//    chunk and serves both token sub-tiles.
//  * Per super-block (256 k) the workgroup stages, with 16-byte buffer loads (hardware
//    range checks give zeros past the last token / row, no branches), the raw qs bytes
//    (128 B per row) and the q8_1 int8 tile into XOR-swizzled LDS, and decodes the block
//    headers once into per-(row, sub-block) f32 terms.
//  * Integer stage: one v_mfma_i32_32x32x32_i8 per (sub-tile, chunk). K = 32 is exactly
//    one q8_1 block and one q4_K sub-block, so no two scales share an integer
//    accumulator. One 16-byte LDS read of raw qs serves two chunks: low nibbles
//    (& 0x0F0F0F0F) are chunk 2p, high nibbles (>> 4 & 0x0F0F0F0F) chunk 2p+1.
//  * The MFMA accumulates onto the bits of 1.5*2^23, so its int32 result read as f32 is
//    1.5*2^23 + I exactly (|I| <= 15*127*32 < 2^22). e = fma(F, da, -1.5*2^23*da) is
//    round(da*I) (the constant is exact: da has 11 significant bits), and
//    y = fma(e, dsv, y) accumulates: two VALU ops per output per chunk, nothing else.
//    MFMAs are issued one step ahead of the fold that consumes them, so the matrix core
//    runs while the VALU folds the previous result.
//  * Min term: per super-block, sum_s m_js * (da*ssum)_is is a K=8 product. m (0..63) is
//    exact in bf16; da*ssum is an exact f32 (11 + 12 significant bits) split into three
//    bf16 pieces that sum to it exactly. Two v_mfma_f32_32x32x16_bf16 (pieces x1|x2 in the
//    two k-groups, then x3 with the second group zeroed) give R with f32 accumulation, and
//    one FMA with -dmin per output and super-block folds it into y. (On gfx950 matrix-core
//    and VALU time add up, so this two-MFMA form is cheaper than carrying -dmin*m through
//    more MFMAs.)
//  * The "isums" instantiation runs the same staging, unpack and MFMA code and stores the
//    integer sums instead of folding them (the bit-exact witness of the integer stage).
#include "qpg_common.h"

namespace qpg {
namespace q4k {

typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64;            // tokens per workgroup tile
constexpr int TN = 128;           // weight rows per workgroup tile
constexpr int DA_STRIDE = 20;     // floats per token: per chunk pair p: da_2p, da_2p+1, c0_2p, c0_2p+1 (+pad)
constexpr int PC_STRIDE = 24;     // bf16 per token: three pieces x 8 sub-blocks (per row: m x 8)

struct alignas(16) Smem {
    alignas(16) uint8_t aq[TM * 256];          // q8 tile, granule g of token t at 16*(g ^ (t & 15))
    alignas(16) uint8_t bq[TN * 128];          // raw qs, granule g of row j at 16*(g ^ ((j >> 1) & 7))
    alignas(16) float bdsv[8][TN];             // d*sc per chunk, rows in C-register order per wave
    alignas(16) float ada[TM * DA_STRIDE];     // da and -1.5*2^23*da per token and chunk
    alignas(16) uint16_t ax[TM * PC_STRIDE];   // bf16 pieces of da*ssum per token
    alignas(16) uint16_t bw[TN * PC_STRIDE];   // m per row and sub-block as bf16 (slots 0..7)
    alignas(16) float bnd[TN];                 // -dmin per row, rows in C-register order per wave
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

// Position of weight row jj (0..31 inside a wave's rows) in C-register order: k-group
// (jj >> 2) & 1 holds registers r = 4*(jj >> 3) + (jj & 3).
__device__ __forceinline__ int c_pos(int jj) { return 16 * ((jj >> 2) & 1) + 4 * (jj >> 3) + (jj & 3); }

__device__ __forceinline__ void split3_bf16(float v, uint16_t* dst, int stride)
{
    // v = b1 + b2 + b3 exactly for v with <= 24 significant bits
    const uint32_t b1 = f32_to_bf16_bits(v);
    const float r1 = v - bf16_bits_to_f32(b1);
    const uint32_t b2 = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(b2);
    const uint32_t b3 = f32_to_bf16_bits(r2);
    dst[0] = (uint16_t)b1;
    dst[stride] = (uint16_t)b2;
    dst[2 * stride] = (uint16_t)b3;
}

template <bool ISUMS>
__global__ void __launch_bounds__(256, ISUMS ? 1 : 3) mmq_q4K_kernel(const uint8_t* __restrict__ W,
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
    const int wrow = nsb * Q4K_BYTES;

    // Buffer descriptors over this tile's rows only: loads past the last token / weight
    // row of the matrix fall outside num_records and return zeros.
    const int rows_w = min(TN, N - n0), rows_t = min(TM, M - m0);
    const __amdgpu_buffer_rsrc_t rW =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (size_t)n0 * wrow), 0, rows_w * wrow, 0x00020000);
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

    const int wr = 32 * wave + l32;                 // weight row of this lane's A operand
    const int wsw = (wr >> 1) & 7;                   // its LDS swizzle
    int tk[2], tsw[2];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
        tk[ts] = 32 * ts + l32;                      // token of this lane's B operand / outputs
        tsw[ts] = tk[ts] & 15;
    }

    for (int sb = 0; sb < nsb; ++sb) {
        // ---------------- stage A: q8 tile (64 tokens x 256 B)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int g = it * 256 + tid, t = g >> 4, gi = g & 15;
            const int32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rQ, t * K + sb * QK_K + gi * 16, 0, 0);
            *reinterpret_cast<int32x4*>(sm.aq + t * 256 + 16 * (gi ^ (t & 15))) = v;
        }
        // ---------------- stage A: headers -> da, -1.5*2^23*da, bf16 pieces of da*ssum
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int h = it * 256 + tid, t = h >> 3, c = h & 7;
            const uint32_t hw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rH, (t * nc + sb * 8 + c) * 4, 0, 0);
            const float da = half_bits_to_float(hw & 0xFFFFu);
            float* ad = sm.ada + t * DA_STRIDE + 4 * (c >> 1) + (c & 1);
            ad[0] = da;
            ad[2] = -MAGIC_F * da;                                  // exact
            split3_bf16(da * (float)(int16_t)(hw >> 16), sm.ax + t * PC_STRIDE + c, 8);   // da*ssum exact
        }
        // ---------------- stage B: raw qs (128 rows x 128 B)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int g = it * 256 + tid, j = g >> 3, gi = g & 7;
            const int32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rW, j * wrow + sb * Q4K_BYTES + 16 + gi * 16, 0, 0);
            *reinterpret_cast<int32x4*>(sm.bq + j * 128 + 16 * (gi ^ ((j >> 1) & 7))) = v;
        }
        // ---------------- stage B: d, dmin and the eight 6-bit (sc, m) pairs of each row
        if (tid < TN) {
            const int j = tid;
            const int32x4 hv = __builtin_amdgcn_raw_buffer_load_b128(rW, j * wrow + sb * Q4K_BYTES, 0, 0);
            const float d = half_bits_to_float((uint32_t)hv[0] & 0xFFFFu);
            const float dmin = half_bits_to_float((uint32_t)hv[0] >> 16);
            const uint32_t S0 = (uint32_t)hv[1], S1 = (uint32_t)hv[2], S2 = (uint32_t)hv[3];
            const int pos = 32 * (j >> 5) + c_pos(j & 31);
            sm.bnd[pos] = -dmin;
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
                sm.bdsv[s][pos] = d * (float)sc;                      // exact (17 bits)
                sm.bw[j * PC_STRIDE + s] = (uint16_t)(__float_as_uint((float)m) >> 16);
            }
        }
        __syncthreads();

        // ---------------- integer stage + fold, MFMA one step ahead of the fold
        // Step k = 0..15 is (chunk c = k/2, token sub-tile ts = k%2). In step k the wave
        // issues the LDS reads for step k+1, the MFMA of step k+1, then folds step k; the
        // scheduling barriers keep that order, so only two accumulator blocks and one set
        // of operands are live at a time.
        auto a_from = [&](const uint32x4& raw, int c) -> int32x4 {
            const uint32x4 u = (c & 1) ? ((raw >> 4u) & 0x0F0F0F0Fu) : (raw & 0x0F0F0F0Fu);
            int32x4 r;
            __builtin_memcpy(&r, &u, 16);
            return r;
        };
        auto ld_raw = [&](int p) -> uint32x4 {
            return *reinterpret_cast<const uint32x4*>(sm.bq + wr * 128 + 16 * ((2 * p + hg) ^ wsw));
        };
        auto ld_b = [&](int c, int ts) -> int32x4 {
            return *reinterpret_cast<const int32x4*>(sm.aq + tk[ts] * 256 + 16 * ((2 * c + hg) ^ tsw[ts]));
        };

        uint32x4 raw = ld_raw(0);
        int32x16 F[2];
        F[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_from(raw, 0), ld_b(0, 0), magic, 0, 0, 0);
        floatx4 dsv[4];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int c = k >> 1, ts = k & 1;
            const int k1 = k + 1, c1 = k1 >> 1, ts1 = k1 & 1;
            int32x4 bn;
            if (k1 < 16) {
                if ((k1 & 3) == 0) raw = ld_raw(k1 >> 2);
                bn = ld_b(c1, ts1);
            }
            if constexpr (!ISUMS) {
                if (ts == 0) {
                    const floatx4* dsvp = reinterpret_cast<const floatx4*>(&sm.bdsv[c][32 * wave + 16 * hg]);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) dsv[q4] = dsvp[q4];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (k1 < 16)
                F[k1 & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_from(raw, c1), bn, magic, 0, 0, 0);
            const int32x16 Fk = F[k & 1];
            if constexpr (ISUMS) {
                const int tok = m0 + tk[ts];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = n0 + 32 * wave + c_row(r, lane);
                    if (tok < M && row < N)
                        S[((size_t)tok * N + row) * nc + sb * 8 + c] = Fk[r] - MAGIC_BITS;
                }
            } else {
                const floatx4 dc = *reinterpret_cast<const floatx4*>(sm.ada + tk[ts] * DA_STRIDE + 4 * (c >> 1));
                const float da = dc[c & 1], c0 = dc[2 + (c & 1)];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * q4 + e;
                        const float ev = fmaf(__int_as_float(Fk[r]), da, c0);       // round(da * I)
                        y[ts][r] = fmaf(ev, dsv[q4][e], y[ts][r]);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---------------- min term: R = sum_s m_s * (x1 + x2 + x3)_s on the matrix core, then
        // y += -dmin * R. MFMA 1 pairs x1 (k-group 0) and x2 (k-group 1) with m, MFMA 2 pairs x3
        // with m in k-group 0 only.
        if constexpr (!ISUMS) {
            const uint16_t* bwr = sm.bw + wr * PC_STRIDE;       // m of this lane's weight row
            bf16x8 mA, mA2;
            __builtin_memcpy(&mA, bwr, 16);
            const int32x4 z4 = {0, 0, 0, 0};
            int32x4 mraw; __builtin_memcpy(&mraw, bwr, 16);
            const int32x4 mraw2 = hg ? z4 : mraw;
            __builtin_memcpy(&mA2, &mraw2, 16);
            floatx4 ndv[4];
            const floatx4* ndp = reinterpret_cast<const floatx4*>(&sm.bnd[32 * wave + 16 * hg]);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) ndv[q4] = ndp[q4];
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                const uint16_t* axr = sm.ax + tk[ts] * PC_STRIDE;
                bf16x8 x12, x3;
                __builtin_memcpy(&x12, axr + 8 * hg, 16);
                __builtin_memcpy(&x3, axr + 16, 16);
                floatx16 R = {};
                R = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mA, x12, R, 0, 0, 0);
                R = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mA2, x3, R, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) y[ts][r] = fmaf(R[r], ndv[r >> 2][r & 3], y[ts][r]);
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
