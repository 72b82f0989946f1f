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
//  * Staging is a two-deep pipeline of half super-blocks (128 k: 8 KiB of q8 tile, 8 KiB
//    of raw qs) moved by LDS-direct buffer loads (buffer_load_dwordx4 ... lds): the loads
//    of stage h+1 are issued before stage h is computed, land in LDS without passing
//    through registers, and are waited for only at the next stage boundary. Each lane
//    fetches the 16-byte granule that belongs at its LDS slot: rows are unpadded, and the
//    source offsets permute the granules of a row so that LDS reads spread over the banks
//    (layout below); tokens / rows past the end of the matrix read an out-of-range offset,
//    which the buffer load returns as zeros. The block
//    headers (q8_1 words, q4_K d/dmin/scales) are loaded into registers one super-block
//    ahead and decoded once per super-block into per-(row, sub-block) and per-(token,
//    chunk) f32 terms.
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
//    exact in bf16; da*ssum (an exact f32 of up to 23 significant bits) enters as two bf16
//    pieces, its top 8 bits (truncation) and the remainder rounded to nearest, which sum to
//    it within 2^-16 of its magnitude (exactly when it has at most 16 significant bits). One
//    v_mfma_f32_32x32x16_bf16 per token sub-tile (pieces x1 | x2 in the two k-groups against
//    m | m) gives R with f32 accumulation, and one FMA with -dmin per output and super-block
//    folds it into y.
//  * The "isums" instantiation runs the same staging, unpack and MFMA code and stores the
//    integer sums instead of folding them (the bit-exact witness of the integer stage).
#include "qpg_common.h"

namespace qpg {
namespace q4k {

typedef unsigned uint32x4 __attribute__((ext_vector_type(4)));
typedef unsigned uint32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int TN = 128;           // weight rows per workgroup tile
constexpr int PC_STRIDE = 16;     // bf16 per token: two pieces x 8 sub-blocks
constexpr int HALF = 128;         // k per pipeline stage (half a super-block)

// LDS of one group of four waves (one K range of the tile). Stage-buffer layouts, in
// 16-byte slots, rows unpadded and the granules of a row permuted so that the 16 consecutive
// tokens / rows of one ds_read_b128 phase fall on 16 distinct 16-byte bank groups (the
// permutation is applied by the LDS-direct loads' per-lane source offsets):
//   q8 tile: token t, granule g (k 16g..16g+15 of the half) at slot 8t + (g ^ ((t >> 1) & 7))
//   raw qs:  row j, granule g (qs bytes 16g.. of the half)   at slot 4j + (g ^ ((j >> 2) & 3))
// TS = token sub-tiles of 32 per wave: the workgroup tile is TM = 32*TS tokens x 128 rows
// (TS = 2 for long prompts, TS = 1 halves the token padding of short ones).
constexpr int BQ_SLOTS = TN * 4;                                  // raw qs: 8 slabs of 64
template <int TS>
struct GroupLds {
    static constexpr int TM = 32 * TS, AQ_SLOTS = TM * 8;         // q8 tile: 4*TS slabs of 64
    alignas(16) uint8_t aq0[AQ_SLOTS * 16];
    alignas(16) uint8_t aq1[AQ_SLOTS * 16];
    alignas(16) uint8_t bq0[BQ_SLOTS * 16];
    alignas(16) uint8_t bq1[BQ_SLOTS * 16];
    alignas(16) float dsv[8][TN];            // d*sc per chunk, rows in C-register order per wave
    alignas(16) float2 ada[8][TM];           // (da, -1.5*2^23*da) per chunk and token
    alignas(16) uint16_t ax[TM * PC_STRIDE]; // bf16 pieces of da*ssum per token
    alignas(16) uint16_t bw[TN * 8];         // m per row and sub-block as bf16
    alignas(16) float bnd[TN];               // -dmin per row, rows in C-register order per wave
};
static_assert(sizeof(GroupLds<2>) == 45568 && sizeof(GroupLds<1>) == 34304, "LDS of one group");
static_assert(4 * (GroupLds<1>::AQ_SLOTS + BQ_SLOTS) * 16 / 2 >= 32 * TN * 4 &&
                  4 * (GroupLds<2>::AQ_SLOTS + BQ_SLOTS) * 16 / 2 >= 64 * TN * 4,
              "a group's stage buffers hold its partial tile");


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

// Position of weight row jj (0..31 inside a wave's rows) in C-register order: k-group
// (jj >> 2) & 1 holds registers r = 4*(jj >> 3) + (jj & 3).
__device__ __forceinline__ int c_pos(int jj) { return 16 * ((jj >> 2) & 1) + 4 * (jj >> 3) + (jj & 3); }

// Wait until this wave's outstanding vector-memory operations (the LDS-direct loads) are
// complete: vmcnt(0), expcnt and lgkmcnt left at their maxima.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One LDS-direct load: each lane's 16 bytes at voff go to LDS byte lds_wave_base + 16*lane.
// Written as inline asm so that the compiler does not track it: its own wait insertion
// can make unrelated LDS reads of the stage being computed wait for the prefetch.
// Completion is waited for explicitly (wait_vmem) before the barrier that publishes the
// stage. The LDS base must be wave-uniform: it is the m0 operand of the instruction, bound
// to that register by the "{m0}" constraint, so the compiler writes m0 itself and knows
// that the statement reads it.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, int voff)
{
    const unsigned la = (unsigned)(uintptr_t)(lds_void*)lds_wave_base;
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(la) : "memory");
}

// KS = number of four-wave groups per workgroup; group g computes the tile over its own
// contiguous range of super-blocks and the partial sums are added in group order at the end.
template <bool ISUMS, int KS, int TS>
__global__ void __launch_bounds__(256 * KS, KS > 1 ? 1 : 3) mmq_q4K_kernel(const uint8_t* __restrict__ W,
                                                         const int8_t* __restrict__ qplane,
                                                         const uint32_t* __restrict__ hdr,
                                                         float* __restrict__ Y,
                                                         int32_t* __restrict__ S,
                                                         int M, int N, int K, int tiles_m, int total, int pieces)
{
    constexpr int TM = 32 * TS;
    __shared__ GroupLds<TS> lds_all[KS];
    int m_tile, n_tile, piece;
    tile_coords(m_tile, n_tile, piece, tiles_m, total, pieces);
    // K-split over workgroups (few tiles): piece p adds the super-blocks [p*nsb/P, (p+1)*nsb/P)
    // and writes its partial tile to Y + p*M*N (a workspace the caller sums in piece order).
    if (pieces > 1) Y += (size_t)piece * M * N;
    const int grp = KS > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8) : 0;
    GroupLds<TS>& L = lds_all[grp];
    const int tid = threadIdx.x & 255, lane = tid & 63;        // thread index inside the group
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Per-lane source offsets of the LDS-direct loads. A slab is 64 consecutive slots
    // (1 KiB) written by one wave instruction, lane L to slot 64*slab + L; the lane fetches
    // the granule that the permutation puts there. The q8 tile has 4*TS slabs, the raw qs 8;
    // wave w loads slabs w, w + 4, ... of both. Stage offsets are added per load.
    unsigned voA[TS], voB[2];
#pragma unroll
    for (int i = 0; i < TS; ++i) {
        const int sl = 64 * (wave + 4 * i) + lane;
        const int t = sl >> 3, ga = (sl & 7) ^ ((t >> 1) & 7);
        voA[i] = (unsigned)(t * K + 16 * ga);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int sl = 64 * (wave + 4 * i) + lane;
        const int j = sl >> 2, gb = (sl & 3) ^ ((j >> 2) & 3);
        voB[i] = (unsigned)(j * wrow + 16 + 16 * gb);
    }

    // The stage offset moves the descriptors' base (scalar arithmetic) instead of every
    // lane's offset; the range shrinks by the same amount, so the bounds are unchanged.
    const int8_t* const qbase = qplane + (size_t)m0 * K;
    const uint8_t* const wbase = W + (size_t)n0 * wrow;
    const unsigned nQ = (unsigned)(rows_t * K), nW = (unsigned)(rows_w * wrow);
    auto issue_stage = [&](int sb, int hh, uint8_t* aq, uint8_t* bq) {
        const unsigned oa = __builtin_amdgcn_readfirstlane(sb * QK_K + hh * HALF);
        const unsigned ob = __builtin_amdgcn_readfirstlane(sb * Q4K_BYTES + hh * (HALF / 2));
        const __amdgpu_buffer_rsrc_t rQs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(qbase + oa), 0, (int)(nQ - oa), 0x00020000);
        const __amdgpu_buffer_rsrc_t rWs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(wbase + ob), 0, (int)(nW - ob), 0x00020000);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i < TS) lds_load16(rQs, aq + 1024 * (wave + 4 * i), (int)voA[i]);
            lds_load16(rWs, bq + 1024 * (wave + 4 * i), (int)voB[i]);
        }
    };

    // Block headers of one super-block, one 16-byte load per thread into registers:
    // threads 0..127 the q4_K header (d, dmin, 12 scale bytes) of row tid, threads
    // 128..255 four q8_1 words (token (tid-128)/2, chunks 4*(tid&1)..+3; with TM = 32 the
    // threads of tokens 32..63 load past the tile's rows, i.e. zeros, and decode nothing).
    auto load_headers = [&](int sb) -> uint32x4 {
        int32x4 v;
        if (tid < TN)
            v = __builtin_amdgcn_raw_buffer_load_b128(rW, tid * wrow + sb * Q4K_BYTES, 0, 0);
        else {
            const int u = tid - TN;
            v = __builtin_amdgcn_raw_buffer_load_b128(rH, ((u >> 1) * nc + sb * 8 + 4 * (u & 1)) * 4, 0, 0);
        }
        return __builtin_bit_cast(uint32x4, v);
    };

    int32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; ++r) magic[r] = MAGIC_BITS;
    floatx16 y[TS];
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[a][r] = 0.0f;

    const int wr = 32 * wave + l32;                 // weight row of this lane's A operand
    // Lane offsets of the compute-phase reads (the token sub-tile is an immediate, +4096):
    // q8 granule 2 cl + hg of token l32 for each chunk cl of a stage, raw granule 2 p + hg of
    // row wr for p = 0, 1.
    int aq_off[4], bq_off[2];
#pragma unroll
    for (int cl = 0; cl < 4; ++cl) aq_off[cl] = 128 * l32 + 16 * ((2 * cl + hg) ^ ((l32 >> 1) & 7));
#pragma unroll
    for (int p = 0; p < 2; ++p) bq_off[p] = 64 * wr + 16 * ((2 * p + hg) ^ ((wr >> 2) & 3));

    // Decode one super-block's headers (held in registers by the thread that loaded them)
    // into the fold terms.
    auto decode_headers = [&](const uint32x4 hv) {
        if (tid < TN) {
            // bytewise unpack of the 12 packed bytes: byte s of each word is sub-block s (s < 4)
            // or s + 4 (the high nibbles of S2 plus the top two bits of S0 / S1)
            const int j = tid;
            const float d = half_bits_to_float(hv[0] & 0xFFFFu);
            const float dmin = half_bits_to_float(hv[0] >> 16);
            const uint32_t S0 = hv[1], S1 = hv[2], S2 = hv[3];
            const uint32_t sc03 = S0 & 0x3F3F3F3Fu, m03 = S1 & 0x3F3F3F3Fu;
            const uint32_t sc47 = (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u);
            const uint32_t m47 = ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u);
            const int pos = 32 * (j >> 5) + c_pos(j & 31);
            L.bnd[pos] = -dmin;
            uint32_t mb[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t scw = s < 4 ? sc03 : sc47, mw = s < 4 ? m03 : m47;
                const int b = 8 * (s & 3);
                L.dsv[s][pos] = d * (float)((scw >> b) & 0xFFu);           // exact (17 bits)
                mb[s] = __float_as_uint((float)((mw >> b) & 0xFFu));         // exact bf16 in the high half
            }
            const uint32x4 mw4 = {(mb[0] >> 16) | (mb[1] & 0xFFFF0000u), (mb[2] >> 16) | (mb[3] & 0xFFFF0000u),
                                  (mb[4] >> 16) | (mb[5] & 0xFFFF0000u), (mb[6] >> 16) | (mb[7] & 0xFFFF0000u)};
            *reinterpret_cast<uint32x4*>(L.bw + j * 8) = mw4;
        } else if (((tid - TN) >> 1) < TM) {
            // per chunk: da, -1.5*2^23*da, and da*ssum as two bf16 pieces: its top 8 significant
            // bits by truncation, then the (exact) remainder rounded to nearest
            const int u = tid - TN, t = u >> 1, c4 = 4 * (u & 1);
            uint32_t p1[4], p2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t hw = hv[e];
                const float da = half_bits_to_float(hw & 0xFFFFu);
                L.ada[c4 + e][t] = make_float2(da, -MAGIC_F * da);        // exact
                const float v = da * (float)(int)(int16_t)(hw >> 16);       // da*ssum exact (23 bits)
                const float b1 = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
                const float r1 = v - b1;                                     // exact
                p1[e] = __float_as_uint(b1);
                p2[e] = f32_to_bf16_bits(r1) << 16;                          // |r1 - p2| <= 2^-16 |v|
            }
            uint16_t* axr = L.ax + t * PC_STRIDE + c4;
            *reinterpret_cast<uint32x2*>(axr) = uint32x2{(p1[0] >> 16) | (p1[1] & 0xFFFF0000u), (p1[2] >> 16) | (p1[3] & 0xFFFF0000u)};
            *reinterpret_cast<uint32x2*>(axr + 8) = uint32x2{(p2[0] >> 16) | (p2[1] & 0xFFFF0000u), (p2[2] >> 16) | (p2[3] & 0xFFFF0000u)};
        }
    };

    // Integer stage + fold over the four chunks of one half super-block, MFMA one step
    // ahead of the fold. Step k = 0..4*TS-1 is (chunk c = 4*hh + k/TS, token sub-tile k%TS);
    // one 16-byte read of raw qs serves 2*TS steps (two chunks).
    auto compute_stage = [&](int sb, int hh, const uint8_t* aq, const uint8_t* bq) {
        auto a_from = [&](const uint32x4& raw, int c) -> int32x4 {
            const uint32x4 u = (c & 1) ? ((raw >> 4u) & 0x0F0F0F0Fu) : (raw & 0x0F0F0F0Fu);
            int32x4 r;
            __builtin_memcpy(&r, &u, 16);
            return r;
        };
        auto ld_raw = [&](int p) -> uint32x4 {
            return *reinterpret_cast<const uint32x4*>(bq + bq_off[p]);
        };
        auto ld_b = [&](int cl, int ts) -> int32x4 {
            return *reinterpret_cast<const int32x4*>(aq + aq_off[cl] + 4096 * ts);
        };
        if constexpr (!ISUMS) asm volatile("" : "+v"(magic));   // keep the constant in VGPRs
        constexpr int NSTEP = 4 * TS;
        uint32x4 raw = ld_raw(0);
        int32x16 F[2];
        F[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_from(raw, 0), ld_b(0, 0), magic, 0, 0, 0);
        floatx4 dsv[4];
#pragma unroll
        for (int k = 0; k < NSTEP; ++k) {
            const int cl = k / TS, ts = k % TS, c = 4 * hh + cl;
            const int k1 = k + 1, cl1 = k1 / TS, ts1 = k1 % TS;
            int32x4 bn;
            if (k1 < NSTEP) {
                if ((k1 % (2 * TS)) == 0) raw = ld_raw(k1 / (2 * TS));
                bn = ld_b(cl1, ts1);
            }
            if constexpr (!ISUMS) {
                if (ts == 0) {
                    const floatx4* dsvp = reinterpret_cast<const floatx4*>(&L.dsv[c][32 * wave + 16 * hg]);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) dsv[q4] = dsvp[q4];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (k1 < NSTEP)
                F[k1 & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_from(raw, cl1), bn, magic, 0, 0, 0);
            const int32x16 Fk = F[k & 1];
            if constexpr (ISUMS) {
                const int tok = m0 + 32 * ts + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = n0 + 32 * wave + c_row(r, lane);
                    if (tok < M && row < N)
                        S[((size_t)tok * N + row) * nc + sb * 8 + c] = Fk[r] - MAGIC_BITS;
                }
            } else {
                const float2 dc = L.ada[c][32 * ts + l32];
                const float da = dc.x, c0 = dc.y;
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
        // The folds of this stage are done here: without the pin, they may be sunk past the
        // next barrier, which keeps all the stage's MFMA results live at once.
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) asm volatile("" : "+v"(y[ts]));
    };

    // Min term of one super-block: R = sum_s m_s * (x1 + x2)_s on the matrix core (x1 in
    // k-group 0, x2 in k-group 1, both against m), then y += -dmin * R.
    auto min_term = [&]() {
        const uint16_t* bwr = L.bw + wr * 8;            // m of this lane's weight row
        bf16x8 mA;
        __builtin_memcpy(&mA, bwr, 16);
        floatx4 ndv[4];
        const floatx4* ndp = reinterpret_cast<const floatx4*>(&L.bnd[32 * wave + 16 * hg]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) ndv[q4] = ndp[q4];
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const uint16_t* axr = L.ax + (32 * ts + l32) * PC_STRIDE;
            bf16x8 x12;
            __builtin_memcpy(&x12, axr + 8 * hg, 16);
            floatx16 R = {};
            R = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mA, x12, R, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) y[ts][r] = fmaf(R[r], ndv[r >> 2][r & 3], y[ts][r]);
        }
    };

    // Pipeline. Stage (sb, 0) lives in buffer 0, (sb, 1) in buffer 1; the loads of the next
    // stage go to the buffer that the barrier just freed. The headers of super-block sb+1
    // are loaded into registers while sb is computed.
    // This group's super-blocks: [sb0, sb0 + cnt). Every group runs the same number of
    // iterations (all waves of the workgroup meet at each barrier); a group with one
    // super-block fewer idles through its last one.
    const int pb0 = (int)(((int64_t)piece * nsb) / pieces), pcnt = (int)(((int64_t)(piece + 1) * nsb) / pieces) - pb0;
    const int nbase = pcnt / KS, nrem = pcnt % KS;
    const int cnt = nbase + (grp < nrem ? 1 : 0), sb0 = pb0 + grp * nbase + min(grp, nrem);
    const int iters = nbase + (nrem ? 1 : 0);
    uint32x4 hv;
    if (cnt > 0) {
        hv = load_headers(sb0);
        issue_stage(sb0, 0, L.aq0, L.bq0);
    }
    // With one group per workgroup (several workgroups per CU), the waits, barriers, header
    // decode and load issue of each half run at wave priority 1 and the compute at 0: a
    // workgroup's short serial section then takes the issue slots ahead of the other
    // workgroups' folds, so fewer of its waves idle at the barriers (1.5-2 % on the
    // 512 x 11008 x 4096 and 1024 x 11008 x 4096 shapes; with three groups in one workgroup,
    // where all waves meet at the same barriers, it measured ~1 % slower and is not used).
    for (int it = 0; it < iters; ++it) {
        const bool act = it < cnt, more = it + 1 < cnt;
        const int sb = sb0 + it;
        // ---- first half: wait for (sb, 0) and the headers of sb, decode the headers
        if constexpr (KS == 1) __builtin_amdgcn_s_setprio(1);
        wait_vmem();
        __syncthreads();                    // stage (sb,0) visible; (sb-1,1) and its min term done
        if constexpr (!ISUMS)
            if (act) decode_headers(hv);
        __syncthreads();                    // fold terms of sb visible
        if (more) hv = load_headers(sb + 1);
        if (act) issue_stage(sb, 1, L.aq1, L.bq1);
        if constexpr (KS == 1) __builtin_amdgcn_s_setprio(0);
        if (act) compute_stage(sb, 0, L.aq0, L.bq0);

        // ---- second half
        if constexpr (KS == 1) __builtin_amdgcn_s_setprio(1);
        wait_vmem();
        __syncthreads();                    // stage (sb,1) visible; buffer 0 free
        if (more) issue_stage(sb + 1, 0, L.aq0, L.bq0);
        if constexpr (KS == 1) __builtin_amdgcn_s_setprio(0);
        if (act) {
            compute_stage(sb, 1, L.aq1, L.bq1);
            if constexpr (!ISUMS) min_term();
        }
    }

    if constexpr (!ISUMS && KS > 1) {
        // Partial tiles of groups 1..KS-1 go through their own (now idle) stage buffers;
        // group 0 adds them in group order. Layout: float4 q of sub-tile ts at
        // ((4 ts + q) * 256 + thread) * 16 bytes, consecutive threads consecutive.
        __syncthreads();                    // every group is done with its stage buffers
        if (grp > 0) {
            floatx4* red = reinterpret_cast<floatx4*>(L.aq0);
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[(4 * ts + q) * 256 + tid] = floatx4{y[ts][4 * q], y[ts][4 * q + 1], y[ts][4 * q + 2], y[ts][4 * q + 3]};
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int g2 = 1; g2 < KS; ++g2) {
            const floatx4* red = reinterpret_cast<const floatx4*>(lds_all[g2].aq0);
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
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
        for (int ts = 0; ts < TS; ++ts) {
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

}  // namespace q4k
}  // namespace qpg

namespace {
template <int TS>
hipError_t launch_q4K(const uint8_t* wb, const int8_t* qplane, const uint32_t* hdr, float* y, int32_t* isums,
                      int64_t M, int64_t N, int64_t K, int pieces, hipStream_t s)
{
    using namespace qpg::q4k;
    const int tiles_m = (int)((M + 32 * TS - 1) / (32 * TS));
    const int tiles_n = (int)((N + TN - 1) / TN);
    const int total = tiles_m * tiles_n;
    // At most one tile per CU (256 CUs): split each tile's super-blocks over three
    // four-wave groups, so each SIMD still holds three waves.
    const bool split = total * pieces <= 256 && (K / 256) / pieces >= 3;
    const unsigned grid = (unsigned)(total * pieces);
    if (isums) {
        if (split)
            hipLaunchKernelGGL((mmq_q4K_kernel<true, 3, TS>), dim3(grid), dim3(768), 0, s, wb, qplane, hdr, y, isums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
        else
            hipLaunchKernelGGL((mmq_q4K_kernel<true, 1, TS>), dim3(grid), dim3(256), 0, s, wb, qplane, hdr, y, isums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
    } else {
        if (split)
            hipLaunchKernelGGL((mmq_q4K_kernel<false, 3, TS>), dim3(grid), dim3(768), 0, s, wb, qplane, hdr, y, isums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
        else
            hipLaunchKernelGGL((mmq_q4K_kernel<false, 1, TS>), dim3(grid), dim3(256), 0, s, wb, qplane, hdr, y, isums,
                               (int)M, (int)N, (int)K, tiles_m, total, pieces);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t qpg_launch_mmq_q4K(const void* w, const void* xq, float* y, int32_t* isums, int64_t M, int64_t N,
                              int64_t K, int pieces, hipStream_t s)
{
    const int8_t* qplane = static_cast<const int8_t*>(xq);
    const uint32_t* hdr = reinterpret_cast<const uint32_t*>(qplane + M * K);
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    return qpg_q4K_tile_m(M, N, K) == 32 ? launch_q4K<1>(wb, qplane, hdr, y, isums, M, N, K, pieces, s)
                                         : launch_q4K<2>(wb, qplane, hdr, y, isums, M, N, K, pieces, s);
}
