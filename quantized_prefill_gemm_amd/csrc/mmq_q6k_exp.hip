// Expanded q6_K x q8_1 MMQ kernel for gfx950 (MI355X).
//
// Y[i][j] = sum over 32-wide chunks c of da_ic * d_{j,c/8} * C_ijc,
//   C_ijc = sum_{k in c} (sc_{j,k/16} * (q6_jk - 32)) * q_ik        (exact int32)
// -- the q6_K sum of "r40 - __launch_bounds__(256,3) third resident block" (sec. 5), two
// 16-wide sub-blocks with their own int8 scales per 32-wide q8_1 chunk, regrouped: the
// int8 scale is applied to each weight before the integer product instead of to each
// 16-wide sum after it. The two forms are the same exact integer sum.
//
// A one-time expand pass (q6K_expand) writes every weight as a = sc * (q6 - 32), an integer
// in [-4064, 4096], in two int8 digits a = 64 * hi + lo (hi in [-64, 64], lo in [0, 63]).
// The kernel then needs no per-element decode at all:
//  * Integer stage: per (32x32 sub-tile, chunk) two v_mfma_i32_32x32x32_i8, hi digits and lo
//    digits against the same q8 operand, each onto the bits of 1.5*2^23:
//    FH = 1.5*2^23 + H, FL = 1.5*2^23 + L (|H|, |L| <= 32*64*127 < 2^22), C = 64H + L.
//    The raw path needs two 32x32x16 MFMAs per chunk for the two sub-blocks: the same
//    matrix-core time.
//  * Fold: e = fma(FH, 64*da, -65*1.5*2^23*da) = 64*da*H - 1.5*2^23*da,
//    e2 = fma(FL, da, e) = da*C, y = fma(e2, d, y): three VALU ops per output and chunk
//    (the raw form needs four: two per sub-block). The constants 64*da and
//    65*1.5*2^23*da are exact (da has 11 significant bits); e carries the magnitude of
//    1.5*2^23*da, so its rounding (<= ~da) is the only error beyond the final f32 sums.
//
// MI355X design:
//  * Tile 64 tokens x 64 weight rows: four 32x32 sub-tiles, rows 32*(w&1).. and tokens
//    32*((w>>1)&1).. (weight rows on the MFMA row side: da is one value per lane, d one value
//    per register). Eight waves per tile: waves w and w+4 compute the same sub-tile over
//    chunks 0-1 and 2-3 of every stage and add their partial sums at the end, so two
//    workgroups per CU give four waves per SIMD (121 VGPRs; one 32x32 tile per wave alone
//    would leave two).
//  * Two-deep pipeline of half super-blocks (128 k) with one barrier per stage, all of it
//    moved by LDS-direct loads issued one stage ahead: the q8 tile (8 KiB, 16-byte loads,
//    natural order), the digit image of the stage (17 KiB, a contiguous copy: the expand
//    pass writes the exact LDS layout), the q8_1 header words (dword loads) and the
//    super-block's d per row (256 B).
//  * LDS layouts (per stage):
//      aq: token t at 128 t, 16-byte granule G (k = 16G..16G+15) at slot G ^ ((t >> 1) & 7)
//      ad: row j at 272 j (odd number of 16-byte slots: 16 rows read together hit 16
//          different bank groups), granule G = 4 cl + 2 p + hg (chunk cl, digit plane
//          p = hi / lo, k-group hg) at 16 G, so every read is one base plus an immediate
//      d:  row j at 32 (j >> 5) + c_pos(j & 31), i.e. each lane's 16 rows contiguous.
//  * When the matrix has at most 256 tiles (one per CU), three groups of four waves share a
//    workgroup over contiguous super-block ranges and add their partial tiles in group
//    order through LDS (deterministic).
//  * The "csums" instantiation stores C (the exact integer witness) instead of folding it.
#include <cstddef>

#include "qpg_common.h"

namespace qpg {
namespace q6kx {

typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int TM = 64;
constexpr int TN = 64;
constexpr int HALF = 128;                       // k per pipeline stage
constexpr int AD_PITCH = 272;                   // digit row: 16 granules + one pad granule
constexpr int EXP_STAGE = TN * AD_PITCH;        // digit image of one stage: 17 KiB
constexpr int EXP_D = TN * 4;                   // d per row of the super-block: 256 B
constexpr int EXP_SB = 2 * EXP_STAGE + EXP_D;   // one (tile, super-block) record: 35,072 B

struct StageLds {
    alignas(16) uint8_t aq[TM * HALF];
    alignas(16) uint8_t ad[EXP_STAGE];
    alignas(16) uint32_t hw[4][TM];             // q8_1 header words (fp16 da | ssum) per chunk and token
    alignas(16) float d[TN];
};
struct GroupLds {
    StageLds st[2];
};
static_assert(sizeof(GroupLds) == 2 * (TM * HALF + EXP_STAGE + 4 * TM * 4 + EXP_D), "LDS of one group");
static_assert(3 * sizeof(GroupLds) <= 160 * 1024, "three groups per CU");
static_assert(sizeof(GroupLds) >= TM * TN * 4, "a group's buffers hold its partial tile");

__device__ __forceinline__ int aq_sw(int t) { return (t >> 1) & 7; }
// Position of row jj (0..31 of a 32-row half) in C-register order: lane half hg holds
// registers r = 0..15 of rows 8(r>>2) + 4hg + (r&3) at 16 hg + r.
__device__ __forceinline__ int c_pos(int jj) { return 16 * ((jj >> 2) & 1) + 4 * (jj >> 3) + (jj & 3); }

__device__ __forceinline__ void tile_coords(int& m_tile, int& n_tile, int& piece, int tiles_m, int total,
                                            int pieces)
{
    // Workgroups are dispatched round-robin over the 8 XCDs (bid % 8). Give each XCD a
    // contiguous range of (tile, K-piece) units, M fastest, so the workgroups sharing a
    // weight tile run on one XCD and read it into that XCD's L2 once.
    const int bid = blockIdx.x, units = total * pieces;
    const int xcd = bid & 7, k = bid >> 3;
    const int q = units >> 3, r = units & 7;
    const int t = xcd * q + (xcd < r ? xcd : r) + k;
    const int tile = t % total;
    piece = t / total;
    m_tile = tile % tiles_m;
    n_tile = tile / tiles_m;
}

// Wait for this wave's outstanding vector-memory operations (the LDS-direct loads).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS-direct loads (inline asm, so that the compiler's own waits do not tie unrelated LDS
// reads to them; completion is waited for explicitly before the barrier that publishes
// them): lane L's 4 / 16 bytes at voff go to LDS byte lds_wave_base + 4L / 16L. The
// wave-uniform LDS base is the instruction's m0 operand ("{m0}" constraint: the compiler
// writes m0 itself and knows that the statement reads it).
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, int voff)
{
    const unsigned la = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(la) : "memory");
}
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, int voff)
{
    const unsigned la = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(la) : "memory");
}

// KS groups of 4 waves over contiguous super-block ranges (few tiles), or KW = 2: 8 waves
// on one tile, waves w and w + 4 computing the same sub-tile over chunks 0-1 and 2-3 of each
// stage (four waves per SIMD with two workgroups per CU).
template <bool CSUMS, int KS, int KW>
__global__ void __launch_bounds__(256 * KS * KW, KS > 1 ? 1 : (KW > 1 ? 2 : 3)) mmq_q6K_exp_kernel(
    const uint8_t* __restrict__ WE, const int8_t* __restrict__ qplane, const uint32_t* __restrict__ hdr,
    float* __restrict__ Y, int32_t* __restrict__ S, int M, int N, int K, int tiles_m, int total, int pieces)
{
    static_assert(KS == 1 || KW == 1, "a K split over groups or over waves, not both");
    constexpr int NW = 4 * KW;                      // waves sharing one set of stage buffers
    __shared__ GroupLds lds_all[KS];
    int m_tile, n_tile, piece;
    tile_coords(m_tile, n_tile, piece, tiles_m, total, pieces);
    // K-split over workgroups (few tiles): piece p adds the super-blocks [p*nsb/P, (p+1)*nsb/P)
    // and writes its partial tile to Y + p*M*N (a workspace the caller sums in piece order).
    if (pieces > 1) Y += (size_t)piece * M * N;
    const int grp = KS > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8) : 0;
    GroupLds& G = lds_all[grp];
    const int tid = threadIdx.x & (64 * NW - 1), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave >> 2;                       // chunk half of the stage (KW = 2)
    const int hg = lane >> 5, l32 = lane & 31;
    const int wr0 = 32 * (wave & 1), wt0 = 32 * ((wave >> 1) & 1);
    const int m0 = m_tile * TM, n0 = n_tile * TN;
    const int nsb = K / QK_K, nc = K / QK8;
    const int rows_t = min(TM, M - m0);

    // Sources of this tile: the expanded records (always in range: rows past N are zero
    // there), the q8 rows and header words of its tokens (loads past the last token fall
    // outside the descriptor range and return zeros).
    const uint8_t* const wtile = WE + (size_t)n_tile * nsb * EXP_SB;
    const int8_t* const qbase = qplane + (size_t)m0 * K;
    const uint8_t* const hbase = reinterpret_cast<const uint8_t*>(hdr + (size_t)m0 * nc);
    const unsigned nW = (unsigned)nsb * EXP_SB, nQ = (unsigned)(rows_t * K), nH = (unsigned)(rows_t * nc * 4);

    // Per-lane source offsets. q8 tile: slab i = tokens 8i..8i+7 (8 lanes each), wave w
    // slabs 2w, 2w+1; lane L of slab i = token 8i + (L >> 3) at slot L & 7, which holds
    // granule (L & 7) ^ aq_sw(t). Digits: 17 contiguous slabs of 1 KiB, wave w slabs
    // 4w..4w+3, wave 0 also slab 16. Header words: wave w brings chunk w of the stage,
    // lane = token.
    // (With 8 waves each takes one q8 slab and two digit slabs.)
    constexpr int QS = 8 / NW, DS = 16 / NW;        // q8 / digit slabs per wave
    int voQ[QS];
#pragma unroll
    for (int i = 0; i < QS; ++i) {
        const int t = 8 * (QS * wave + i) + (lane >> 3);
        voQ[i] = t * K + 16 * ((lane & 7) ^ aq_sw(t));
    }
    const int voH = lane * nc * 4 + 4 * (wave & 3);

    // The stage offset moves each descriptor's base (scalar arithmetic) and shrinks its
    // range by the same amount, so the per-lane offsets stay fixed and the bounds unchanged.
    auto issue_stage = [&](int sb, int hh, StageLds& st) {
        const unsigned oq = __builtin_amdgcn_readfirstlane(sb * QK_K + hh * HALF);
        const unsigned ow = __builtin_amdgcn_readfirstlane(sb * EXP_SB + hh * EXP_STAGE);
        const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)(qbase + oq), 0, (int)(nQ - oq), 0x00020000);
        const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)(wtile + ow), 0, (int)(nW - ow), 0x00020000);
#pragma unroll
        for (int i = 0; i < QS; ++i) lds_load16(rQ, st.aq + 1024 * (QS * wave + i), voQ[i]);
#pragma unroll
        for (int i = 0; i < DS; ++i) lds_load16(rW, st.ad + 1024 * (DS * wave + i), 1024 * (DS * wave + i) + 16 * lane);
        if (wave == 0) lds_load16(rW, st.ad + 1024 * 16, 1024 * 16 + 16 * lane);     // 17th slab
        if constexpr (!CSUMS) {
            const unsigned oh = __builtin_amdgcn_readfirstlane((sb * 8 + 4 * hh) * 4);
            const __amdgpu_buffer_rsrc_t rH = __builtin_amdgcn_make_buffer_rsrc((void*)(hbase + oh), 0, (int)(nH - oh), 0x00020000);
            if (wave < 4) lds_load4(rH, &st.hw[wave][0], voH);
            if (wave == 0 && lane < 16) {
                const unsigned od = __builtin_amdgcn_readfirstlane(sb * EXP_SB + 2 * EXP_STAGE);
                const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc((void*)(wtile + od), 0, EXP_D, 0x00020000);
                lds_load16(rD, st.d, 16 * lane);
            }
        }
    };

    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_BITS;
    floatx16 y;
#pragma unroll
    for (int r = 0; r < 16; ++r) y[r] = 0.0f;

    const int jr = wr0 + l32, tt = wt0 + l32;       // A row and B token of this lane
    // Lane offsets of the compute reads (the rest is immediates): A at row jr, k-group hg;
    // B granule (2 cl + hg) ^ aq_sw(tt) of token tt for each chunk cl.
    const int aoff = AD_PITCH * jr + 16 * hg;
    int boff[4];
#pragma unroll
    for (int cl = 0; cl < 4; ++cl) boff[cl] = 128 * tt + 16 * ((2 * cl + hg) ^ aq_sw(tt));

    // Integer stage + fold over the four chunks of one stage, the two MFMAs of chunk cl+1
    // issued before the fold of chunk cl.
    auto compute_stage = [&](int sb, int hh, const StageLds& st) {
        if constexpr (!CSUMS) asm volatile("" : "+v"(magic));   // keep the constant in VGPRs
        auto ldA = [&](int cl, int p) -> int32x4 {
            return *reinterpret_cast<const int32x4*>(st.ad + aoff + 16 * (4 * cl + 2 * p));
        };
        auto ldB = [&](int cl) -> int32x4 { return *reinterpret_cast<const int32x4*>(st.aq + boff[cl]); };
        floatx4 dv[4];
        if constexpr (!CSUMS) {
            const floatx4* dp = reinterpret_cast<const floatx4*>(&st.d[wr0 + 16 * hg]);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) dv[q4] = dp[q4];
        }
        auto fold = [&](int cl, const int32x16& fh, const int32x16& fl) {
            if constexpr (CSUMS) {
                const int tok = m0 + tt;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = n0 + wr0 + c_row(r, lane);
                    if (tok < M && row < N)
                        S[((size_t)tok * N + row) * nc + sb * 8 + 4 * hh + cl] = 64 * (fh[r] - MAGIC_BITS) + (fl[r] - MAGIC_BITS);
                }
            } else {
                float da = half_bits_to_float(st.hw[cl][tt] & 0xFFFFu);
                // an f32 register, so that t2 is a v_fmac_f32 (reading the f16 half directly
                // makes it a mixed-precision v_fma_mix_f32, which issues at ~2/3 the rate)
                asm volatile("" : "+v"(da));
                const float da64 = 64.0f * da, c1 = -65.0f * MAGIC_F * da;          // both exact
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * q4 + e;
                        const float t1 = fmaf(__int_as_float(fh[r]), da64, c1);      // 64 da H - 1.5*2^23 da
                        const float t2 = fmaf(__int_as_float(fl[r]), da, t1);        // da (64 H + L)
                        y[r] = fmaf(t2, dv[q4][e], y[r]);
                    }
            }
        };
        if constexpr (KW > 1) {
            // two chunks per wave; the other waves of the SIMD cover the MFMA latency
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int cl = 2 * kh + x;
                const int32x4 b = ldB(cl);
                const int32x16 fh = __builtin_amdgcn_mfma_i32_32x32x32_i8(ldA(cl, 0), b, magic, 0, 0, 0);
                const int32x16 fl = __builtin_amdgcn_mfma_i32_32x32x32_i8(ldA(cl, 1), b, magic, 0, 0, 0);
                fold(cl, fh, fl);
            }
        } else {
            int32x16 FH[2], FL[2];
            {
                const int32x4 b = ldB(0);
                FH[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ldA(0, 0), b, magic, 0, 0, 0);
                FL[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ldA(0, 1), b, magic, 0, 0, 0);
            }
#pragma unroll
            for (int cl = 0; cl < 4; ++cl) {
                int32x4 bn, ahn, aln;
                if (cl + 1 < 4) {
                    bn = ldB(cl + 1);
                    ahn = ldA(cl + 1, 0);
                    aln = ldA(cl + 1, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (cl + 1 < 4) {
                    FH[(cl + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahn, bn, magic, 0, 0, 0);
                    FL[(cl + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aln, bn, magic, 0, 0, 0);
                }
                fold(cl, FH[cl & 1], FL[cl & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // folds of this stage done here (not sunk past the next barrier)
        asm volatile("" : "+v"(y));
    };

    // Pipeline over this group's stages: super-blocks [sb0, sb0 + cnt), two stages each.
    // Every group runs the same number of stages so that all waves meet at every barrier.
    const int pb0 = (int)(((int64_t)piece * nsb) / pieces), pcnt = (int)(((int64_t)(piece + 1) * nsb) / pieces) - pb0;
    const int nbase = pcnt / KS, nrem = pcnt % KS;
    const int cnt = nbase + (grp < nrem ? 1 : 0), sb0 = pb0 + grp * nbase + min(grp, nrem);
    const int iters = nbase + (nrem ? 1 : 0);
    // Stage (sb, 0) lives in buffer 0 and (sb, 1) in buffer 1, so every LDS address of the
    // compute is a lane offset plus an immediate.
    if (cnt > 0) issue_stage(sb0, 0, G.st[0]);
    for (int it = 0; it < iters; ++it) {
        const int sb = sb0 + it;
        const bool act = it < cnt, more = it + 1 < cnt;
        wait_vmem();
        __syncthreads();                    // stage (sb,0) visible in buffer 0; buffer 1 free
        if (act) issue_stage(sb, 1, G.st[1]);
        if (act) compute_stage(sb, 0, G.st[0]);
        wait_vmem();
        __syncthreads();                    // stage (sb,1) visible in buffer 1; buffer 0 free
        if (more) issue_stage(sb + 1, 0, G.st[0]);
        if (act) compute_stage(sb, 1, G.st[1]);
    }

    if constexpr (!CSUMS && KS > 1) {
        // Partial tiles of groups 1..KS-1 through their own (now idle) LDS; group 0 adds them
        // in group order. float4 q at (q * 256 + thread) * 16 bytes.
        __syncthreads();
        if (grp > 0) {
            floatx4* red = reinterpret_cast<floatx4*>(&G);
#pragma unroll
            for (int q = 0; q < 4; ++q) red[q * 256 + tid] = floatx4{y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g2 = 1; g2 < KS; ++g2) {
            const floatx4* red = reinterpret_cast<const floatx4*>(&lds_all[g2]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const floatx4 p = red[q * 256 + tid];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[4 * q + e] += p[e];
            }
        }
    }

    if constexpr (!CSUMS && KW > 1) {
        // waves 4..7 hand their chunk-half partial sums to waves 0..3, which add them (in
        // that fixed order) and store; layout float4 q at (q * 256 + thread) * 16 bytes
        __syncthreads();                    // every wave is done with the stage buffers
        floatx4* red = reinterpret_cast<floatx4*>(&G);
        if (kh == 1)
#pragma unroll
            for (int q = 0; q < 4; ++q) red[q * 256 + (tid & 255)] = floatx4{y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const floatx4 p = red[q * 256 + tid];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[4 * q + e] += p[e];
        }
    }

    if constexpr (!CSUMS) {
        // lane holds token m0 + tt; register group b = r>>2 holds the four consecutive
        // weight rows n0 + wr0 + 8b + 4hg + 0..3
        const int tok = m0 + tt;
        if (tok < M) {
            const bool vec = ((N & 3) == 0) && ((((uintptr_t)Y) & 15) == 0);
            float* yrow = Y + (size_t)tok * N;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int row = n0 + wr0 + 8 * b + 4 * hg;
                if (vec && row + 3 < N) {
                    *reinterpret_cast<floatx4*>(yrow + row) = floatx4{y[4 * b], y[4 * b + 1], y[4 * b + 2], y[4 * b + 3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (row + e < N) yrow[row + e] = y[4 * b + e];
                }
            }
        }
    }
}

// Expand raw q6_K blocks: workgroup (T, sb), thread (row j = tid & 63, quarter qq = tid >> 6)
// writes the digits of weights 64qq..64qq+63 of row j's block sb (stage qq >> 1, chunks
// 2(qq&1), 2(qq&1)+1), and the qq = 0 threads row j's d. Raw rows are only 2-byte aligned,
// so the block is read bytewise (one pass per matrix).
__global__ void __launch_bounds__(256) q6K_expand_kernel(const uint8_t* __restrict__ W, uint8_t* __restrict__ WE,
                                                         int N, int K)
{
    const int nsb = K / QK_K;
    const size_t wrow = (size_t)nsb * Q6K_BYTES;
    const int T = (int)(blockIdx.x / (unsigned)nsb), sb = (int)(blockIdx.x % (unsigned)nsb);
    const int j = threadIdx.x & 63, qq = threadIdx.x >> 6, n = T * TN + j;
    const int hh = qq >> 1;
    // digits of k = 64qq + 32x + 16g + b (x: chunk of the pair, g: k-group, b: byte)
    uint32_t hi[16], lo[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) hi[i] = lo[i] = 0u;
    float d = 0.0f;
    if (n < N) {
        const uint8_t* blk = W + (size_t)n * wrow + (size_t)sb * Q6K_BYTES;
        const uint8_t* ql = blk;
        const uint8_t* qh = blk + 128;
        const int8_t* sc = reinterpret_cast<const int8_t*>(blk + 192);
#pragma unroll
        for (int kk = 0; kk < 64; ++kk) {
            const int k = 64 * qq + kk;                      // element of the block
            const int h = k >> 7, r = k & 127, g = r >> 5, l = r & 31;
            const int low = (ql[64 * h + 32 * (g & 1) + l] >> (4 * (g >> 1))) & 15;
            const int high = (qh[32 * h + l] >> (2 * g)) & 3;
            const int a = ((low | (high << 4)) - 32) * (int)sc[k >> 4];   // in [-4064, 4096]
            const int dh = a >> 6, dl = a & 63;                          // a = 64 dh + dl
            hi[kk >> 2] |= (uint32_t)(dh & 0xFF) << (8 * (kk & 3));
            lo[kk >> 2] |= (uint32_t)dl << (8 * (kk & 3));
        }
        d = half_bits_to_float((uint32_t)blk[208] | ((uint32_t)blk[209] << 8));
    }
    uint8_t* rec = WE + ((size_t)T * nsb + sb) * EXP_SB;
    uint8_t* row = rec + hh * EXP_STAGE + AD_PITCH * j;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int cl = 2 * (qq & 1) + x, q = 4 * (2 * x + g);       // dword index of the granule
            *reinterpret_cast<uint32x4*>(row + 16 * (4 * cl + 0 + g)) = uint32x4{hi[q], hi[q + 1], hi[q + 2], hi[q + 3]};
            *reinterpret_cast<uint32x4*>(row + 16 * (4 * cl + 2 + g)) = uint32x4{lo[q], lo[q + 1], lo[q + 2], lo[q + 3]};
        }
    if ((qq & 1) == 0) *reinterpret_cast<uint32x4*>(row + 256) = uint32x4{0u, 0u, 0u, 0u};     // pad granule
    if (qq == 0) reinterpret_cast<float*>(rec + 2 * EXP_STAGE)[32 * (j >> 5) + c_pos(j & 31)] = d;
}

}  // namespace q6kx
}  // namespace qpg

hipError_t qpg_launch_q6K_expand(const void* w, void* we, int64_t N, int64_t K, hipStream_t s)
{
    using namespace qpg::q6kx;
    const int64_t tiles_n = (N + TN - 1) / TN;
    hipLaunchKernelGGL(q6K_expand_kernel, dim3((unsigned)(tiles_n * (K / 256))), dim3(256), 0, s,
                       static_cast<const uint8_t*>(w), static_cast<uint8_t*>(we), (int)N, (int)K);
    return hipGetLastError();
}

hipError_t qpg_launch_mmq_q6K_exp(const void* we, const void* xq, float* y, int32_t* csums, int64_t M, int64_t N,
                                  int64_t K, int pieces, hipStream_t s)
{
    using namespace qpg::q6kx;
    const int tiles_m = (int)((M + TM - 1) / TM);
    const int tiles_n = (int)((N + TN - 1) / TN);
    const int total = tiles_m * tiles_n;
    const int8_t* qplane = static_cast<const int8_t*>(xq);
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(qplane + M * K);
    const uint8_t* wb = static_cast<const uint8_t*>(we);
    // At most one tile per CU: split each tile's super-blocks over three groups; otherwise
    // eight waves per tile (two per SIMD) split each stage's chunks.
    const bool split = total * pieces <= 256 && (K / 256) / pieces >= 3;
    const unsigned grid = (unsigned)(total * pieces);
    if (csums) {
        if (split)
            hipLaunchKernelGGL((mmq_q6K_exp_kernel<true, 3, 1>), dim3(grid), dim3(768), 0, s, wb, qplane, hdr, y, csums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
        else
            hipLaunchKernelGGL((mmq_q6K_exp_kernel<true, 1, 2>), dim3(grid), dim3(512), 0, s, wb, qplane, hdr, y, csums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
    } else {
        if (split)
            hipLaunchKernelGGL((mmq_q6K_exp_kernel<false, 3, 1>), dim3(grid), dim3(768), 0, s, wb, qplane, hdr, y, csums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
        else
            hipLaunchKernelGGL((mmq_q6K_exp_kernel<false, 1, 2>), dim3(grid), dim3(512), 0, s, wb, qplane, hdr, y, csums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
    }
    return hipGetLastError();
}
