/*
 * qpg.h -- C ABI of libqpg.so: k-quant mixed-precision matrix multiply (MMQ) for LLM
 * prefill on AMD Instinct MI355X (gfx950).
 *
 *   Y[M][N] (f32) = W[N][K] (q4_K or q6_K blocks) x q8_1(X[M][K] f32)^T
 *
 * The computation is the one of the minfer optimisation log ("r28 - Direction-A
 * raw-nibble NB kernel", sec. 2.3): activations are quantised per 32 values to int8
 * with an fp16 scale and an int16 block sum; each 32-wide (q4_K) or 16-wide (q6_K)
 * sub-block product is an exact integer dot product; the integer sums are folded into
 * f32 with the weight's per-sub-block scale (d*sc) and, for q4_K, the min term
 * (-dmin*m) times the activation block sum.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers of the current HIP device. The caller owns every
 *     buffer; the library allocates and frees nothing, prints nothing and keeps no
 *     state besides per-device caches (device properties; the address of the fixed
 *     scratch of mmq_q4K_noalloc, a device array the runtime places on each device when
 *     the library's code loads there).
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); nothing
 *     synchronises. Buffers must stay valid until the stream reaches the work.
 *   - Shapes: M = tokens, N = output features (weight rows), K = input features.
 *     1 <= M, N; 256 <= K; K % 256 == 0; M, N, K < 2^31.
 *   - Return value: QPG_OK (0) on success, a negative QPG_E* code otherwise. Arguments
 *     and the device are checked before anything is enqueued, so on QPG_EINVAL,
 *     QPG_EALIGN and QPG_EDEVICE nothing has been. QPG_EHIP reports a failed kernel
 *     launch; in the entry points that enqueue two kernels (mmq_q4K / mmq_q6K: quantise,
 *     then the MMQ; the _sk entry points with a split: the MMQ, then the reduce) the first
 *     may already be enqueued when the second fails. QPG_ESCRATCH (mmq_q4K_noalloc only)
 *     is reported before anything is enqueued. There is no fallback path.
 *   - The library runs on gfx950 only (QPG_EDEVICE otherwise).
 *
 * Data layouts
 *   q4_K weights: row-major, row j = K/256 consecutive 144-byte super-blocks:
 *       +0 fp16 d, +2 fp16 dmin, +4 12 bytes of packed 6-bit (scale, min) pairs for the
 *       eight 32-weight sub-blocks, +16 128 bytes qs (4-bit quants; byte 32p + l holds
 *       element l of sub-block 2p in its low nibble and of sub-block 2p+1 in its high
 *       nibble). Weight = d*sc_s*nib - dmin*m_s. (GGUF q4_K; the 144-byte stride and the
 *       qs placement are the ones of "r28", sec. 3.2, and "r29 - NB kd-loop unroll",
 *       sec. 3.2.) Pointer must be 16-byte aligned.
 *   q6_K weights: row-major, row j = K/256 consecutive 210-byte super-blocks:
 *       +0 ql[128] low 4 bits, +128 qh[64] high 2 bits, +192 int8 scales[16] (one per
 *       16 weights), +208 fp16 d. Weight = d*sc[e/16]*(q6 - 32). (GGUF q6_K.) Pointer
 *       must be 2-byte aligned (the block's own alignment: its fp16 d). The MMQ kernels
 *       stage the blocks by byte-addressed direct-to-LDS loads, so row and block starts
 *       need no more; q6K_prepare alone asks for 4 bytes.
 *   q8_1 activations ("xq"), one buffer of qpg_q8_1_bytes(M, K) bytes, two planes:
 *       bytes [0, M*K):            int8 q[M][K], row-major
 *       bytes [M*K, M*K + 4*M*K/32): uint32 header[M][K/32]; low 16 bits = fp16 scale
 *                                  d of the 32-value block, high 16 bits = int16 sum
 *                                  of its 32 q values (the pages' "d | ssum" word).
 *       Pointer must be 16-byte aligned.
 *   X (f32 [M][K] row-major, 16-byte aligned) and Y (f32 [M][N] row-major, 4-byte
 *   aligned; overwritten, never accumulated into).
 */
#ifndef QPG_H
#define QPG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qpg_stream_t;   /* hipStream_t */

enum {
    QPG_OK = 0,
    QPG_EINVAL = -1,   /* null pointer, bad shape (M/N < 1, K % 256, too large)   */
    QPG_EALIGN = -2,   /* a pointer violates its alignment requirement           */
    QPG_EHIP = -3,     /* the HIP runtime reported an error when enqueuing        */
    QPG_EDEVICE = -4,  /* current device is not gfx950 or cannot be queried       */
    QPG_ESCRATCH = -5  /* more than the fixed scratch of mmq_q4K_noalloc needed   */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* qpg_strerror(int status);

/* Size in bytes of the q8_1 buffer for an M x K activation: M*K + 4*M*(K/32).
 * Returns 0 when M < 1, K < 32 or K % 32 != 0. */
size_t qpg_q8_1_bytes(int64_t M, int64_t K);

/*
 * quantize_q8_1: X f32 [M][K] -> xq (q8_1 layout above).
 * Per 32-value block: amax = max|x|; d = amax / 127 (IEEE f32 division);
 * q = round(x * (1/d)) with 1/d an IEEE f32 division and ties rounded away from zero
 * (q = 0 when d = 0); sum = sum of the 32 q; stored scale = fp16(d), round to nearest
 * even. The q values use the unrounded f32 d. Non-finite inputs are outside the
 * contract. (q8_1 header: "r28", sec. 3.2 smem map; the rounding rule is a reading.)
 * Here K needs only K % 32 == 0.
 */
int quantize_q8_1(const float* x, void* xq, int64_t M, int64_t K, qpg_stream_t stream);

/*
 * mmq_q4K / mmq_q6K: Y = W x q8_1(X)^T from f32 activations. Enqueues quantize_q8_1
 * into the caller's workspace xq_ws (qpg_q8_1_bytes(M, K) bytes, 16-byte aligned),
 * then the MMQ kernel (same as the _q8 entry points). On return of the stream, xq_ws
 * holds q8_1(X).
 * q4_K: Y[i][j] = sum_c da_ic*(d*sc)_jc*I_ijc + da_ic*ssum_ic*(-dmin*m)_jc, with
 *       I_ijc = sum of nib*q over the 32 k of chunk c (exact int32)   ("r28", sec. 2.3)
 * q6_K: Y[i][j] = sum_u da_{i,u/2}*(d*sc)_ju*J_iju, J = 16-wide int32 sums
 *       ("r40 - third resident block", sec. 5: two 16-k products per 32-k chunk)
 * The f32 summation order is the kernel's own; results agree with the exact value to
 * |err| <= 1e-4*|y| + 1e-3*rms(Y).
 */
int mmq_q4K(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
            void* xq_ws, qpg_stream_t stream);
int mmq_q6K(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
            void* xq_ws, qpg_stream_t stream);

/*
 * mmq_q4K_noalloc: mmq_q4K without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The q8_1 activations go to a fixed device array of
 * QPG_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every device it runs on
 * until the process ends; the call itself allocates nothing. Shapes whose q8_1 buffer,
 * qpg_q8_1_bytes(M, K), exceeds the array are refused with QPG_ESCRATCH before anything
 * is enqueued (e.g. M * K <= 29.8 M values: 2048 x 11008 or 4096 x 4096 fit). Same result
 * as mmq_q4K, bit for bit. The first call on a device looks up the array's device address
 * (a host-side runtime query, no stream work); make it outside graph capture. All calls
 * on one device share its array and the last call's q8_1 data stays in it: calls that
 * overlap in time on one device (two streams, two threads) race and must be serialised
 * by the caller. Alignment: w, x 16 bytes; y 4 bytes.
 */
#define QPG_NOALLOC_SCRATCH_BYTES (32u << 20)
int mmq_q4K_noalloc(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
                    qpg_stream_t stream);

/* The MMQ kernels alone, on an already quantised q8_1 buffer xq. */
int mmq_q4K_q8(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
               qpg_stream_t stream);
int mmq_q6K_q8(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
               qpg_stream_t stream);

/*
 * Integer stage only: the same staging, unpack and int8 MFMA code as the _q8 entry
 * points, writing the exact int32 sub-block sums instead of folding them.
 *   mmq_q4K_isums: s int32 [M][N][K/32], s[i][j][c] = I_ijc
 *   mmq_q6K_isums: s int32 [M][N][K/16], s[i][j][u] = J_iju
 * s must be 4-byte aligned; M*N*(K/16) must be < 2^40 elements.
 */
int mmq_q4K_isums(const void* w, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                  qpg_stream_t stream);
int mmq_q6K_isums(const void* w, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                  qpg_stream_t stream);

/*
 * Prepared q6_K weights (the q6_K "prepare" pass of "r41"-"r53" in the pages' NEXT
 * list: a one-time repack into an aligned layout that the kernel stages with plain 16-byte
 * direct-to-LDS copies). q6K_prepare reads raw q6_K blocks w [N][K/256] (4-byte aligned)
 * and writes wp (qpg_q6K_prep_bytes(N, K) bytes, 16-byte aligned, caller-owned): per
 * 128-row tile and super-block two 16 KiB stage images holding the ql / qh bytes
 * (reordered and swizzled) and d*sc[u] as f32 (exact). The layout is library-internal:
 * wp is only meaningful to the _prep entry points of the same library, and must be
 * prepared again after w changes. Rows past N are zero-filled.
 * mmq_q6K_prep_q8 / mmq_q6K_prep_isums compute exactly what mmq_q6K_q8 / mmq_q6K_isums
 * compute from the raw blocks (the integer sums are identical; outputs agree to the
 * same tolerance). qpg_q6K_prep_bytes returns 0 for an unsupported shape
 * (N < 1, K % 256 != 0, K > 2^24 - 256).
 */
size_t qpg_q6K_prep_bytes(int64_t N, int64_t K);
int q6K_prepare(const void* w, void* wp, int64_t N, int64_t K, qpg_stream_t stream);
int mmq_q6K_prep_q8(const void* wp, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                    qpg_stream_t stream);
int mmq_q6K_prep_isums(const void* wp, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                       qpg_stream_t stream);

/*
 * Expanded q6_K weights: a one-time pass that applies each weight's int8 sub-block scale
 * in the integer domain. The q6_K sum of "r40 - __launch_bounds__(256,3) third resident
 * block" (sec. 5) has two 16-wide products per 32-wide q8_1 chunk, each with its own scale
 * sc[u]; sum_u sc[u] * J_u is the same exact integer as sum_k (sc[k/16] * (q6_k - 32)) * q_k,
 * so q6K_expand stores a = sc * (q6 - 32) (in [-4064, 4096]) per weight as two int8 digits
 * (a = 64 * hi + lo) and the kernel forms the chunk sum with two K = 32 int8 products and a
 * three-operation fold. q6K_expand reads raw q6_K blocks w [N][K/256] (any alignment) and
 * writes we (qpg_q6K_exp_bytes(N, K) bytes = ceil(N/64) * (K/256) * 35,072, 16-byte aligned,
 * caller-owned; 2.14 bytes per weight against 0.82 for the raw blocks): per 64-row tile and
 * super-block the two digit planes of both half super-blocks and d as f32. The layout is
 * library-internal: we is only meaningful to the _exp entry points of the same library and
 * must be expanded again after w changes. Rows past N are zero-filled.
 * mmq_q6K_exp_q8 computes what mmq_q6K_q8 computes (same tolerance against the exact
 * result). mmq_q6K_exp_csums writes the exact integer chunk sums
 * s[M][N][K/32] (int32, row-major, caller-owned): s[i][j][c] = sum over k in chunk c of
 * sc[j][k/16] * (q6[j][k] - 32) * q[i][k] -- bit-exact, the witness of the integer stage.
 * qpg_q6K_exp_bytes returns 0 for an unsupported shape (N < 1, K % 256 != 0,
 * K > 2^24 - 256). Alignment: we, xq 16 bytes; y, s 4 bytes. Errors as above; nothing is
 * allocated.
 */
size_t qpg_q6K_exp_bytes(int64_t N, int64_t K);
int q6K_expand(const void* w, void* we, int64_t N, int64_t K, qpg_stream_t stream);
int mmq_q6K_exp_q8(const void* we, const void* xq, float* y, int64_t M, int64_t N, int64_t K,
                   qpg_stream_t stream);
int mmq_q6K_exp_csums(const void* we, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                      qpg_stream_t stream);

/*
 * K split over workgroups, for shapes with few output tiles (a tensor-parallel shard, a
 * short prompt against a narrow matrix): the same sums as the entry points without _sk
 * (mmq_q4K_q8, mmq_q6K_q8, mmq_q6K_prep_q8, mmq_q6K_exp_q8; same operands, alignment and
 * tolerance), with the super-block range of each output tile cut into P contiguous pieces
 * that run as separate workgroups. Each piece writes its partial tile to plane p of the
 * caller's workspace ws (f32 [P][M][N]); a second kernel then sums the planes in piece
 * order into y, so the result is deterministic and independent of scheduling.
 * qpg_mmq_sk_bytes(M, N, K, form) gives the workspace size in bytes (form 0 q4_K, 1 q6_K,
 * 2 prepared q6_K, 3 expanded q6_K): P*M*N*4, or 0 when the shape needs no split (more
 * than 128 output tiles, or too few super-blocks for two pieces) or is unsupported; with 0,
 * ws may be null and the call is the plain entry point. Tiles are 64 tokens x 128 rows
 * (64 x 64 for form 3; q4_K uses 32-token tiles where its 64 x 128 grid has <= 128 tiles).
 * P is at most 8; when all M tokens fit one tile height, P <= 512 / tiles with >= 1
 * super-block per piece, otherwise P <= 256 / tiles with >= 3 per piece. ws must be 16-byte
 * aligned and at least that large (QPG_EINVAL otherwise); it is caller-owned scratch whose
 * contents are overwritten. Calls that share ws must not overlap in time.
 */
size_t qpg_mmq_sk_bytes(int64_t M, int64_t N, int64_t K, int form);
int mmq_q4K_q8_sk(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                  size_t ws_bytes, qpg_stream_t stream);
int mmq_q6K_q8_sk(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                  size_t ws_bytes, qpg_stream_t stream);
int mmq_q6K_prep_q8_sk(const void* wp, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                       size_t ws_bytes, qpg_stream_t stream);
int mmq_q6K_exp_q8_sk(const void* we, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                      size_t ws_bytes, qpg_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QPG_H */
