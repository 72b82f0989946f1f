// q6_K x q8_1 MMQ kernel for gfx950 (MI355X).
//
// Y[i][j] = sum over 16-wide sub-blocks u of da_{i,u/2} * (d*sc)_{ju} * J_iju,
//   J_iju = sum_{k in u} (q6_jk - 32) * q_ik  (exact int32).
// q6_K carries one int8 scale per 16 weights, so each 32-wide q8_1 chunk holds two
// integer products with different scales -- the two 16-k products per 32-k chunk of the
// q6_K kernel of "r40 - __launch_bounds__(256,3) third resident block" (sec. 5).
//
// MI355X design:
//  * Tile 64 tokens x 128 weight rows per group of 4 waves; wave w = weight rows
//    32w..32w+31 (MFMA row side) x 64 tokens (two 32x32 sub-tiles on the column side):
//    da is one value per lane, d*sc is read once per sub-block for both token sub-tiles.
//  * Integer stage: v_mfma_i32_32x32x16_i8 per (token sub-tile, 16-wide sub-block). The
//    weight operand v = q6 - 32 is assembled per byte in registers from the raw ql / qh bytes
//    in LDS: q6 = low4 + (high2 << 4), and v = (q6 + 0x60) ^ 0x80 turns the unsigned 6-bit
//    value into the signed int8 q6 - 32 with no carry between bytes (q6 + 96 <= 159).
//  * The MFMA accumulates onto the bits of 1.5*2^23, so its int32 result read as f32 is
//    1.5*2^23 + J exactly (|J| <= 32*127*16 < 2^22): e = fma(F, da, -1.5*2^23*da) is
//    round(da*J) and y = fma(e, d*sc, y). Two VALU ops per output and sub-block.
//  * Staging is a two-deep pipeline of half super-blocks (128 k, one barrier per stage),
//    all of it by LDS-direct loads issued one stage ahead: the q8 tile by 16-byte loads
//    (buffer_load_dwordx4 ... lds) in natural order, the q8_1 header words by dword loads,
//    and the raw weight bytes by 16-byte loads straight from the blocks. A lane's source
//    offset may be any byte offset (rows of 210-byte blocks start only 2-byte aligned when
//    K/256 is odd), so rows need no register staging and no shifts; the per-lane offsets
//    apply the row swizzle. Each wave loads exactly its own 32 weight rows, and with the first
//    stage of a super-block their 16 int8 scales and d (one 16-byte and one dword load of 32
//    lanes, a row each: rows are far apart, so a load costs by the rows it touches), so after
//    its own load wait it converts their d*sc for both stages without another barrier; the
//    barrier is for the q8 tile and header words, which every wave reads.
//  * LDS: rows of the ql and qh halves XOR-swizzled in 16-byte granules (reads of 16
//    consecutive rows hit 16 bank groups). A K=16 MFMA wants k-group l>>5 of its sub-block in
//    lane l: 8 bytes of each of the chunk's two sub-blocks. The prepared form (q6K_prepare:
//    this stage layout written once to memory, with d*sc included, staged by plain 16-byte
//    copies) swaps the 8-byte pieces 1 and 2 of every 32-byte group, so one 16-byte read gives
//    a lane both; on raw blocks the lane halves read the two sub-blocks' granules and
//    exchange the middle pieces with v_permlane32_swap (two per chunk). The matching q8
//    operand is two 8-byte reads.
//  * When the matrix has at most one tile per CU, three groups of four waves share a
//    workgroup, each over a contiguous range of super-blocks, and the partial tiles are
//    added in group order through LDS at the end (three waves per SIMD, deterministic).
#include <cstddef>

#include "qpg_common.h"

namespace qpg {
namespace q6k {

typedef unsigned uint32x2 __attribute__((ext_vector_type(2)));
typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int TM = 64;
constexpr int TN = 128;
constexpr int HALF = 128;          // k per pipeline stage

// One pipeline stage (half a super-block) of one group.
//   aq:  token t at 128 t; granule G (16 consecutive k) at slot G ^ ((t >> 1) & 7)
//   bl:  ql half, row j at 64 j; granule G (group G>>1, part G&1) at slot G ^ ((j >> 2) & 3)
//   bh:  qh half, row j at 32 j; granule G at slot G ^ ((j >> 3) & 1)
struct StageLds {
    alignas(16) uint8_t aq[TM * HALF];
    alignas(16) uint8_t bl[TN * 64];
    alignas(16) uint8_t bh[TN * 32];
    alignas(16) float dsc[8][TN];       // d*sc per sub-block of the stage, rows in C-register order per wave
    alignas(16) uint32_t hw[4][TM];     // q8_1 header words (fp16 da | ssum) per chunk of the stage and token
};
struct GroupLds {
    StageLds st[2];
    // raw blocks, per wave and super-block, as loaded: the 16 int8 scales of each of the wave's
    // 32 rows (4 words per row), then the word holding fp16 d (block bytes 206..209, d in the
    // high half) of each row
    alignas(16) uint32_t wsd[4][32 * 4 + 32];
};
static_assert(sizeof(GroupLds) == 53760, "LDS of one group");
static_assert(3 * sizeof(GroupLds) <= 160 * 1024, "three groups per CU");
static_assert(sizeof(GroupLds) >= TM * TN * 4, "a group's buffers hold its partial tile");

__device__ __forceinline__ int aq_sw(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int bl_sw(int j) { return (j >> 2) & 3; }
__device__ __forceinline__ int bh_sw(int j) { return (j >> 3) & 1; }

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

__device__ __forceinline__ int c_pos(int jj) { return 16 * ((jj >> 2) & 1) + 4 * (jj >> 3) + (jj & 3); }

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One dword LDS-direct load: each lane's 4 bytes at voff go to LDS byte lds_wave_base + 4*lane.
// Inline asm, so that the compiler's own waits do not tie unrelated LDS reads to it;
// completion is waited for explicitly (wait_vmem) before the barrier that publishes it.
// The wave-uniform LDS base is the instruction's m0 operand ("{m0}" constraint: the
// compiler writes m0 itself and knows that the statement reads it).
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, int voff)
{
    const unsigned la = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(la) : "memory");
}

// 16-byte form of the same load: lane L's 16 bytes at voff go to LDS byte lds_wave_base + 16L.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, int voff)
{
    const unsigned la = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(la) : "memory");
}

// Prepared q6_K weights: per 128-row tile T and super-block sb, two 16 KiB stage images
// (stage hh = weights 128hh..128hh+127 of the super-block) at ((T * nsb + sb) * 2 + hh) *
// 16 KiB, each laid out exactly as StageLds::bl | bh | dsc (contiguous there): the ql half
// and the qh half with the 8-byte piece swap and the row swizzle applied, then d*sc of the
// stage's 8 sub-blocks in C-register row order. Rows past N are zero.
constexpr int PREP_STAGE = 16384;
static_assert(offsetof(StageLds, bh) == offsetof(StageLds, bl) + TN * 64 &&
                  offsetof(StageLds, dsc) == offsetof(StageLds, bh) + TN * 32 &&
                  sizeof(StageLds::bl) + sizeof(StageLds::bh) + sizeof(StageLds::dsc) == PREP_STAGE,
              "stage image = bl | bh | dsc");

// PREP: W is the prepared layout (16-byte aligned, no register staging, the q8 tile in
// natural order by 16-byte loads and its operands read as two 8-byte halves).
template <bool ISUMS, int KS, bool PREP>
__global__ void __launch_bounds__(256 * KS, KS > 1 ? 1 : 3) mmq_q6K_kernel(
    const uint8_t* __restrict__ W, const int8_t* __restrict__ qplane, const uint32_t* __restrict__ hdr,
    float* __restrict__ Y, int32_t* __restrict__ S, int M, int N, int K, int tiles_m, int total, int pieces)
{
    __shared__ GroupLds lds_all[KS];
    int m_tile, n_tile, piece;
    tile_coords(m_tile, n_tile, piece, tiles_m, total, pieces);
    // K-split over workgroups (few tiles): piece p adds the super-blocks [p*nsb/P, (p+1)*nsb/P)
    // and writes its partial tile to Y + p*M*N (a workspace the caller sums in piece order).
    if (pieces > 1) Y += (size_t)piece * M * N;
    const int grp = KS > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8) : 0;
    GroupLds& G = lds_all[grp];
    const int tid = threadIdx.x & 255, lane = tid & 63;        // thread index inside the group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hg = lane >> 5, l32 = lane & 31;
    const int m0 = m_tile * TM, n0 = n_tile * TN;
    const int nsb = K / QK_K, nc = K / QK8, nu = K / 16;
    const int wrow = nsb * Q6K_BYTES;

    // Buffer descriptors over this tile's rows: loads past the last token / weight row
    // return zeros.
    const int rows_w = min(TN, N - n0), rows_t = min(TM, M - m0);
    const __amdgpu_buffer_rsrc_t rW = PREP
        ? __builtin_amdgcn_make_buffer_rsrc((void*)(W + (size_t)n_tile * nsb * 2 * PREP_STAGE), 0, nsb * 2 * PREP_STAGE,
                                            0x00020000)
        : __builtin_amdgcn_make_buffer_rsrc((void*)(W + (size_t)n0 * wrow), 0, rows_w * wrow, 0x00020000);
    const __amdgpu_buffer_rsrc_t rQ =
        __builtin_amdgcn_make_buffer_rsrc((void*)(qplane + (size_t)m0 * K), 0, rows_t * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rH =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hdr + (size_t)m0 * nc), 0, rows_t * nc * 4, 0x00020000);

    // q8_1 header words of the stage: wave w brings chunk w of the stage, lane = token.
    const int voH = lane * nc * 4 + 4 * wave;
    // The q8 tile in natural order by 16-byte loads, slab i = tokens 8i..8i+7 (8 lanes
    // each), wave w slabs 2w, 2w+1; granule G of token t at slot G ^ aq_sw(t). Prepared
    // weights: the stage image, 16 slabs of 1 KiB, wave w slabs 4w..4w+3.
    int voQ16[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = 8 * (2 * wave + i) + (lane >> 3);
        voQ16[i] = t * K + 16 * ((lane & 7) ^ aq_sw(t));
    }
    // Raw blocks: the stage's bytes go straight into LDS by 16-byte LDS-direct loads (a lane
    // may read at any byte offset: rows of 210-byte blocks start 2-byte aligned). ql: LDS slot
    // sl = row sl >> 2, slot sl & 3 holds the row's 16-byte granule (sl & 3) ^ bl_sw(row) of its
    // stage half; qh: row sl >> 1, granule (sl & 1) ^ bh_sw(row). A slab is 64 slots (1 KiB);
    // wave w loads ql slabs 2w, 2w + 1 and qh slab w, i.e. exactly its own 32 rows, and the
    // scales and d of those rows.
    unsigned voL[2], voB = 0, voS = 0;
    if constexpr (!PREP) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int sl = 64 * (2 * wave + i) + lane;          // ql slot: row sl >> 2, slot sl & 3
            const int j = sl >> 2;
            voL[i] = (unsigned)(j * wrow + 16 * ((sl & 3) ^ bl_sw(j)));
        }
        {
            const int sl = 64 * wave + lane;                     // qh slot: row sl >> 1, slot sl & 1
            const int j = sl >> 1;
            voB = (unsigned)(j * wrow + 16 * ((sl & 1) ^ bh_sw(j)));
        }
        voS = (unsigned)((32 * wave + (lane & 31)) * wrow);     // lanes 0..31: row 32 wave + lane
    }
    const uint8_t* const wbase = W + (size_t)n0 * wrow;
    const unsigned nW = (unsigned)(rows_w * wrow);
    // A descriptor over this tile's rows starting at byte `off` of every row's first block
    // (the stage offset moves the base and shrinks the range by the same amount, so loads
    // of rows past N still fall outside it and read zeros).
    auto wdesc = [&](unsigned off) {
        off = __builtin_amdgcn_readfirstlane(off);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(wbase + off), 0, (int)(nW - off), 0x00020000);
    };
    auto issue_stage = [&](int sb, int hh, StageLds& st) {
        const int off = sb * QK_K + hh * HALF;
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_load16(rQ, st.aq + 1024 * (2 * wave + i), voQ16[i] + off);
        if constexpr (PREP) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_load16(rW, st.bl + 1024 * (4 * wave + i), (sb * 2 + hh) * PREP_STAGE + 1024 * (4 * wave + i) + 16 * lane);
        } else {
            const unsigned blk = (unsigned)(sb * Q6K_BYTES);
            const __amdgpu_buffer_rsrc_t rL = wdesc(blk + 64 * hh), rB = wdesc(blk + 128 + 32 * hh);
#pragma unroll
            for (int i = 0; i < 2; ++i) lds_load16(rL, st.bl + 1024 * (2 * wave + i), (int)voL[i]);
            lds_load16(rB, st.bh + 1024 * wave, (int)voB);
            // the scales and d of the super-block, once (with its first stage): 32 lanes, one row
            // each, 16 bytes of scales and the word holding d
            if (!ISUMS && hh == 0 && lane < 32) {
                lds_load16(wdesc(blk + 192), &G.wsd[wave][0], (int)voS);
                lds_load4(wdesc(blk + 206), &G.wsd[wave][128], (int)voS);
            }
        }
        if constexpr (!ISUMS) lds_load4(rH, &st.hw[wave][0], voH + (sb * 8 + 4 * hh) * 4);
    };
    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_BITS;
    floatx16 y[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[a][r] = 0.0f;

    const int wr = 32 * wave + l32;                  // weight row of this lane's A operand
    const int tsw = aq_sw(l32);                      // tokens l32 and l32 + 32 share the swizzle

    // d*sc of this wave's 32 rows for all 16 sub-blocks of the super-block, from the scales and
    // d the wave loaded itself (so only its own load wait is needed), at its first stage: lane
    // (jj, half) converts the eight scales of stage `half` of row 32 wave + jj into that stage's
    // buffer (the other buffer's d*sc was last read by this wave's own previous stage).
    auto decode_dsc = [&]() {
        const int jj = l32;
        const uint32_t* sw = &G.wsd[wave][4 * jj + 2 * hg];
        const uint32_t s0 = sw[0], s1 = sw[1];
        const float d = half_bits_to_float(G.wsd[wave][128 + jj] >> 16);
        const int pos = 32 * wave + c_pos(jj);
        StageLds& st = G.st[hg];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            st.dsc[e][pos] = d * (float)(int)(int8_t)((e < 4 ? s0 : s1) >> (8 * (e & 3)));   // exact
    };

    // Integer stage + fold over the four chunks of one stage (chunk cl = sub-blocks 2cl and
    // 2cl+1 of the stage = sub-blocks 8hh + 2cl, +1 of the super-block).
    auto compute_stage = [&](int sb, int hh, const StageLds& st) {
        const uint32x4 qh = *reinterpret_cast<const uint32x4*>(st.bh + 32 * wr + 16 * (hg ^ bh_sw(wr)));
#pragma unroll
        for (int cl = 0; cl < 4; ++cl) {
            __builtin_amdgcn_sched_barrier(0);
            const uint32x4 ql = *reinterpret_cast<const uint32x4*>(st.bl + 64 * wr + 16 * ((2 * (cl & 1) + hg) ^ bl_sw(wr)));
            uint32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = (ql[e] >> (4 * (cl >> 1))) & 0x0F0F0F0Fu;
                // bits 2cl, 2cl+1 of each qh byte moved to bits 4, 5
                const uint32_t hs = cl < 2 ? qh[e] << (4 - 2 * cl) : qh[e] >> (2 * cl - 4);
                const uint32_t hi = hs & 0x30303030u;
                // q6 = lo + hi <= 63 per byte; q6 + 96 <= 159 never carries into the next byte,
                // and (q6 + 96) ^ 0x80 is the signed byte q6 - 32
                v[e] = (lo + hi + 0x60606060u) ^ 0x80808080u;
            }
            if constexpr (!PREP) {
                // raw order: lane half hg holds all 16 bytes of sub-block 2cl + hg; exchange the
                // middle 8-byte pieces between the halves (upper half's dwords 0-1 <-> lower
                // half's dwords 2-3), so each half holds its k-group of both sub-blocks
                const auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
                v[0] = s0[0];
                v[2] = s0[1];
                v[1] = s1[0];
                v[3] = s1[1];
            }
            const long a0 = (long)(((unsigned long)v[1] << 32) | v[0]);      // sub-block 2cl, k-group hg
            const long a1 = (long)(((unsigned long)v[3] << 32) | v[2]);      // sub-block 2cl+1
#pragma unroll
            for (int ts = 0; ts < 2; ++ts) {
                __builtin_amdgcn_sched_barrier(0);
                // natural order: piece hg in granule 2cl, piece 2+hg in granule 2cl+1
                const uint8_t* row = st.aq + 128 * (32 * ts + l32) + 8 * hg;
                const long b0 = *reinterpret_cast<const long*>(row + 16 * ((2 * cl) ^ tsw));
                const long b1 = *reinterpret_cast<const long*>(row + 16 * ((2 * cl + 1) ^ tsw));
                const int32x16 F0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a0, b0, magic, 0, 0, 0);
                const int32x16 F1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a1, b1, magic, 0, 0, 0);
                if constexpr (ISUMS) {
                    const int tok = m0 + 32 * ts + l32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = n0 + 32 * wave + c_row(r, lane);
                        if (tok < M && row < N) {
                            int32_t* dst = S + ((size_t)tok * N + row) * nu + sb * 16 + 8 * hh + 2 * cl;
                            dst[0] = F0[r] - MAGIC_BITS;
                            dst[1] = F1[r] - MAGIC_BITS;
                        }
                    }
                } else {
                    float da = half_bits_to_float(st.hw[cl][32 * ts + l32] & 0xFFFFu);
                    // an f32 register, so the fold is v_fma_f32 (a mixed-precision v_fma_mix_f32
                    // reading the f16 half directly issues at ~2/3 the rate)
                    asm volatile("" : "+v"(da));
                    const float c0 = -MAGIC_F * da;                                       // exact
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int32x16 Fs = s ? F1 : F0;
                        const floatx4* dp = reinterpret_cast<const floatx4*>(&st.dsc[2 * cl + s][32 * wave + 16 * hg]);
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const floatx4 d4 = dp[q4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int r = 4 * q4 + e;
                                const float ev = fmaf(__int_as_float(Fs[r]), da, c0);    // round(da * J)
                                y[ts][r] = fmaf(ev, d4[e], y[ts][r]);
                            }
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // folds of this stage done here (not sunk past the next barrier)
        asm volatile("" : "+v"(y[0]), "+v"(y[1]));
    };

    // Pipeline over this group's stages: super-blocks [sb0, sb0 + cnt), two stages each.
    // Every group runs the same number of stages so that all waves meet at every barrier.
    const int pb0 = (int)(((int64_t)piece * nsb) / pieces), pcnt = (int)(((int64_t)(piece + 1) * nsb) / pieces) - pb0;
    const int nbase = pcnt / KS, nrem = pcnt % KS;
    const int cnt = nbase + (grp < nrem ? 1 : 0), sb0 = pb0 + grp * nbase + min(grp, nrem);
    const int nst = 2 * cnt, nst_all = 2 * (nbase + (nrem ? 1 : 0));
    if (nst > 0) issue_stage(sb0, 0, G.st[0]);
    for (int h = 0; h < nst_all; ++h) {
        const int sb = sb0 + (h >> 1), hh = h & 1, cur = h & 1;
        wait_vmem();
        __syncthreads();                    // stage h visible in buffer cur; buffer cur^1 free
        if (h + 1 < nst) issue_stage(sb0 + ((h + 1) >> 1), (h + 1) & 1, G.st[cur ^ 1]);
        if (h < nst) {
            if constexpr (!PREP && !ISUMS)
                if (hh == 0) decode_dsc();
            compute_stage(sb, hh, G.st[cur]);
        }
    }

    if constexpr (!ISUMS && KS > 1) {
        // Partial tiles of groups 1..KS-1 through their own (now idle) LDS; group 0 adds
        // them in group order. float4 q of sub-tile ts at ((4 ts + q) * 256 + thread) * 16.
        __syncthreads();
        if (grp > 0) {
            floatx4* red = reinterpret_cast<floatx4*>(&G);
#pragma unroll
            for (int ts = 0; ts < 2; ++ts)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[(4 * ts + q) * 256 + tid] = floatx4{y[ts][4 * q], y[ts][4 * q + 1], y[ts][4 * q + 2], y[ts][4 * q + 3]};
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g2 = 1; g2 < KS; ++g2) {
            const floatx4* red = reinterpret_cast<const floatx4*>(&lds_all[g2]);
#pragma unroll
            for (int ts = 0; ts < 2; ++ts)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx4 p = red[(4 * ts + q) * 256 + tid];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[ts][4 * q + e] += p[e];
                }
        }
    }

    if constexpr (!ISUMS) {
        // lane (ts, l32) holds token m0 + 32ts + l32; register group b = r>>2 holds the four
        // consecutive weight rows n0 + 32*wave + 8b + 4hg + 0..3
        const bool vec = ((N & 3) == 0) && ((((uintptr_t)Y) & 15) == 0);
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {
            const int tok = m0 + 32 * ts + l32;
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

// Repack raw q6_K blocks into the prepared layout: workgroup (T, sb), thread (row j =
// tid & 127, stage hh = tid >> 7) writes row j's part of stage image hh. Rows start only
// 2-byte aligned, so the bytes are read as aligned dwords and shifted with v_alignbyte.
__global__ void __launch_bounds__(256) q6K_prepare_kernel(const uint8_t* __restrict__ W, uint8_t* __restrict__ WP,
                                                          int N, int K)
{
    const int nsb = K / QK_K, wrow = nsb * Q6K_BYTES;
    const int T = (int)(blockIdx.x / (unsigned)nsb), sb = (int)(blockIdx.x % (unsigned)nsb);
    const int j = threadIdx.x & 127, hh = threadIdx.x >> 7, n = T * TN + j;
    uint32_t ql[16], qh[8];
    float dsc[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) ql[i] = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) { qh[i] = 0u; dsc[i] = 0.0f; }
    if (n < N) {
        const uint8_t* blk = W + (size_t)n * wrow + (size_t)sb * Q6K_BYTES;
        const uint32_t sh = (uint32_t)((uintptr_t)blk & 2);
        const uint32_t* a = reinterpret_cast<const uint32_t*>(blk + 64 * hh - sh);        // ends by blk + 132
#pragma unroll
        for (int i = 0; i < 16; ++i) ql[i] = __builtin_amdgcn_alignbyte(a[i + 1], a[i], sh);
        const uint32_t* b = reinterpret_cast<const uint32_t*>(blk + 128 + 32 * hh - sh);   // ends by blk + 196
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[i] = __builtin_amdgcn_alignbyte(b[i + 1], b[i], sh);
        const uint32_t* c = reinterpret_cast<const uint32_t*>(blk + 192 + 8 * hh - sh);
        const uint32_t c2 = sh ? c[2] : 0u;                                                  // ends at blk + 210
        const uint32_t s0 = __builtin_amdgcn_alignbyte(c[1], c[0], sh), s1 = __builtin_amdgcn_alignbyte(c2, c[1], sh);
        const float d = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + 208));
#pragma unroll
        for (int u = 0; u < 8; ++u) dsc[u] = d * (float)(int)(int8_t)((u < 4 ? s0 : s1) >> (8 * (u & 3)));   // exact
    }
    uint8_t* img = WP + ((size_t)(T * nsb + sb) * 2 + hh) * PREP_STAGE;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const uint32x4 v = {ql[8 * g + 2 * x], ql[8 * g + 2 * x + 1], ql[8 * g + 4 + 2 * x], ql[8 * g + 5 + 2 * x]};
            *reinterpret_cast<uint32x4*>(img + 64 * j + 16 * ((2 * g + x) ^ bl_sw(j))) = v;
        }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const uint32x4 v = {qh[2 * x], qh[2 * x + 1], qh[4 + 2 * x], qh[5 + 2 * x]};
        *reinterpret_cast<uint32x4*>(img + TN * 64 + 32 * j + 16 * (x ^ bh_sw(j))) = v;
    }
    float* dp = reinterpret_cast<float*>(img + TN * 96);
    const int pos = 32 * (j >> 5) + c_pos(j & 31);
#pragma unroll
    for (int u = 0; u < 8; ++u) dp[u * TN + pos] = dsc[u];
}

}  // namespace q6k
}  // namespace qpg

namespace {
template <bool PREP>
hipError_t launch_q6K(const void* w, const void* xq, float* y, int32_t* isums, int64_t M, int64_t N, int64_t K,
                      int pieces, hipStream_t s)
{
    using namespace qpg::q6k;
    const int tiles_m = (int)((M + TM - 1) / TM);
    const int tiles_n = (int)((N + TN - 1) / TN);
    const int total = tiles_m * tiles_n;
    const int8_t* qplane = static_cast<const int8_t*>(xq);
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(qplane + M * K);
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    // At most one tile per CU (256 CUs): split each tile's super-blocks over three groups.
    const bool split = total * pieces <= 256 && (K / 256) / pieces >= 3;
    const unsigned grid = (unsigned)(total * pieces);
    if (isums) {
        if (split)
            hipLaunchKernelGGL((mmq_q6K_kernel<true, 3, PREP>), dim3(grid), dim3(768), 0, s, wb, qplane, hdr, y,
                               isums, (int)M, (int)N, (int)K, tiles_m, total, pieces);
        else
            hipLaunchKernelGGL((mmq_q6K_kernel<true, 1, PREP>), dim3(grid), dim3(256), 0, s, wb, qplane, hdr, y,
                               isums, (int)M, (int)N, (int)K, tiles_m, total, pieces);
    } else {
        if (split)
            hipLaunchKernelGGL((mmq_q6K_kernel<false, 3, PREP>), dim3(grid), dim3(768), 0, s, wb, qplane, hdr, y,
                               isums, (int)M, (int)N, (int)K, tiles_m, total, pieces);
        else
            hipLaunchKernelGGL((mmq_q6K_kernel<false, 1, PREP>), dim3(grid), dim3(256), 0, s, wb, qplane, hdr, y,
                               isums, (int)M, (int)N, (int)K, tiles_m, total, pieces);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t qpg_launch_mmq_q6K(const void* w, const void* xq, float* y, int32_t* isums, int64_t M, int64_t N,
                              int64_t K, int pieces, hipStream_t s)
{
    return launch_q6K<false>(w, xq, y, isums, M, N, K, pieces, s);
}

hipError_t qpg_launch_mmq_q6K_prep(const void* wp, const void* xq, float* y, int32_t* isums, int64_t M, int64_t N,
                                   int64_t K, int pieces, hipStream_t s)
{
    return launch_q6K<true>(wp, xq, y, isums, M, N, K, pieces, s);
}

hipError_t qpg_launch_q6K_prepare(const void* w, void* wp, int64_t N, int64_t K, hipStream_t s)
{
    using namespace qpg::q6k;
    const int64_t tiles_n = (N + TN - 1) / TN;
    hipLaunchKernelGGL(q6K_prepare_kernel, dim3((unsigned)(tiles_n * (K / 256))), dim3(256), 0, s,
                       static_cast<const uint8_t*>(w), static_cast<uint8_t*>(wp), (int)N, (int)K);
    return hipGetLastError();
}
