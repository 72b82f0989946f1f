// C ABI of libqpg.so (declared in include/qpg.h): argument validation, device check,
// then the kernel launches. Nothing here allocates, frees, prints or synchronises.
#include <mutex>

#include "../../include/qpg.h"
#include "qpg_common.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // M, N < 2^31
constexpr int64_t kMaxK = (int64_t)1 << 24;     // K <= 2^24 keeps every per-tile byte offset < 2^31

// Per-device "is gfx950" cache: 0 unknown, 1 yes, -1 no.
int g_dev_ok[64];
std::mutex g_dev_mu;

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return QPG_EDEVICE;
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_ok[dev] == 0) {
            hipDeviceProp_t p;
            if (hipGetDeviceProperties(&p, dev) != hipSuccess) return QPG_EDEVICE;
            const char* a = p.gcnArchName;
            g_dev_ok[dev] = (a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
                             a[5] == '0' && (a[6] == 0 || a[6] == ':'))
                                ? 1
                                : -1;
        }
        return g_dev_ok[dev] == 1 ? QPG_OK : QPG_EDEVICE;
    }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_mmq_shape(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < 256 || K % 256 != 0) return QPG_EINVAL;
    if (M >= kMaxDim || N >= kMaxDim || K > kMaxK) return QPG_EINVAL;
    // tile counts must fit one grid dimension (counted at the smallest tile, 32 x 128)
    const int64_t tiles = ((M + 31) / 32) * ((N + 127) / 128);
    if (tiles >= kMaxDim) return QPG_EINVAL;
    return QPG_OK;
}

// ---- The allocation-free entry point's scratch: one fixed array per device, holding the q8_1
// activations that mmq_q4K otherwise writes into the caller's workspace. The runtime
// places a copy on every device the library runs on when the code object loads there; it
// lives until the process ends. Host code never passes the array's name to a kernel (on
// the host it names a stand-in, not device memory): the device address of each copy is
// looked up once per device with hipGetSymbolAddress, that device being current, and
// cached.
static __device__ __align__(256) uint8_t scratch[QPG_NOALLOC_SCRATCH_BYTES];
void* g_scratch[64];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return QPG_EDEVICE;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QPG_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return QPG_OK;
}

int status_of(hipError_t e)
{
    if (e == hipSuccess) return QPG_OK;
    return QPG_EHIP;
}

int quantize_checked(const float* x, void* xq, int64_t M, int64_t K, hipStream_t s)
{
    if (!x || !xq) return QPG_EINVAL;
    if (M < 1 || K < 32 || K % 32 != 0 || M >= kMaxDim || K >= kMaxDim) return QPG_EINVAL;
    if ((M * (K / 32) * 8 + 255) / 256 >= kMaxDim) return QPG_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 16)) return QPG_EALIGN;
    const int dv = check_device();
    if (dv != QPG_OK) return dv;
    return status_of(qpg_launch_quantize_q8_1(x, xq, M, K, s));
}

int mmq_checked(bool q6, const void* w, const void* xq, float* y, int32_t* s, int64_t M, int64_t N, int64_t K,
                hipStream_t st)
{
    if (!w || !xq || (!y && !s)) return QPG_EINVAL;
    int rc = check_mmq_shape(M, N, K);
    if (rc != QPG_OK) return rc;
    if (s && M * N * (K / 16) >= ((int64_t)1 << 40)) return QPG_EINVAL;
    if (!aligned(w, q6 ? 2 : 16) || !aligned(xq, 16) || (y && !aligned(y, 4)) || (s && !aligned(s, 4)))
        return QPG_EALIGN;
    rc = check_device();
    if (rc != QPG_OK) return rc;
    return status_of(q6 ? qpg_launch_mmq_q6K(w, xq, y, s, M, N, K, 1, st)
                        : qpg_launch_mmq_q4K(w, xq, y, s, M, N, K, 1, st));
}

// Prepared q6_K: the per-tile record offsets (nsb * 32 KiB) must stay below 2^31.
constexpr int64_t kPrepTile = 128, kPrepSb = 32768;

int prep_shape_ok(int64_t N, int64_t K)
{
    return N >= 1 && N < kMaxDim && K >= 256 && K % 256 == 0 && K <= kMaxK && (K / 256) * kPrepSb < kMaxDim &&
           ((N + kPrepTile - 1) / kPrepTile) * (K / 256) < kMaxDim;
}

int mmq_prep_checked(const void* wp, const void* xq, float* y, int32_t* s, int64_t M, int64_t N, int64_t K,
                     hipStream_t st)
{
    if (!wp || !xq || (!y && !s)) return QPG_EINVAL;
    int rc = check_mmq_shape(M, N, K);
    if (rc != QPG_OK) return rc;
    if (!prep_shape_ok(N, K)) return QPG_EINVAL;
    if (s && M * N * (K / 16) >= ((int64_t)1 << 40)) return QPG_EINVAL;
    if (!aligned(wp, 16) || !aligned(xq, 16) || (y && !aligned(y, 4)) || (s && !aligned(s, 4))) return QPG_EALIGN;
    rc = check_device();
    if (rc != QPG_OK) return rc;
    return status_of(qpg_launch_mmq_q6K_prep(wp, xq, y, s, M, N, K, 1, st));
}

// Expanded q6_K: the per-tile record range (nsb * 35,072 bytes) must stay below 2^31.
constexpr int64_t kExpTile = 64, kExpSb = 35072;

int exp_shape_ok(int64_t N, int64_t K)
{
    return N >= 1 && N < kMaxDim && K >= 256 && K % 256 == 0 && K <= kMaxK && (K / 256) * kExpSb < kMaxDim &&
           ((N + kExpTile - 1) / kExpTile) * (K / 256) < kMaxDim;
}

int mmq_exp_checked(const void* we, const void* xq, float* y, int32_t* s, int64_t M, int64_t N, int64_t K,
                    hipStream_t st)
{
    if (!we || !xq || (!y && !s)) return QPG_EINVAL;
    int rc = check_mmq_shape(M, N, K);
    if (rc != QPG_OK) return rc;
    if (!exp_shape_ok(N, K)) return QPG_EINVAL;
    if (((M + 63) / 64) * ((N + kExpTile - 1) / kExpTile) >= kMaxDim) return QPG_EINVAL;
    if (s && M * N * (K / 32) >= ((int64_t)1 << 40)) return QPG_EINVAL;
    if (!aligned(we, 16) || !aligned(xq, 16) || (y && !aligned(y, 4)) || (s && !aligned(s, 4))) return QPG_EALIGN;
    rc = check_device();
    if (rc != QPG_OK) return rc;
    return status_of(qpg_launch_mmq_q6K_exp(we, xq, y, s, M, N, K, 1, st));
}

// ---- K split over workgroups for shapes with few tiles (at most 128: fewer than half the
// CUs busy). Pieces are contiguous super-block ranges. With several rows of token tiles, each
// piece keeps >= 3 super-blocks (so each of a workgroup's three groups still gets one) and the
// pieces together fill at most one workgroup per CU. With a single row of token tiles (the
// prompt fits one tile height) the call is a stream of the weights with little work per byte:
// pieces of >= 1 super-block, up to two four-wave workgroups per CU, read the weights sooner
// (measured at 16 tokens: 4096 x 4096 q4_K 10.2 -> 8.7 us, expanded q6_K 10.8 -> 10.0 us).
constexpr int kSkMaxPieces = 8;

int64_t form_tile_m(int form, int64_t M, int64_t N, int64_t K)
{
    return form == 0 ? qpg_q4K_tile_m(M, N, K) : 64;               // the q4_K kernel's tile height per shape
}

int64_t form_tiles(int form, int64_t M, int64_t N, int64_t K)
{
    const int64_t tm = form_tile_m(form, M, N, K);
    const int64_t tn = form == 3 ? 64 : 128;                        // expanded q6_K uses 64-row tiles
    return ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
}

int sk_pieces(int form, int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = form_tiles(form, M, N, K);
    if (tiles > 128) return 1;
    const bool one_row = M <= form_tile_m(form, M, N, K);
    int64_t p = (one_row ? 512 : 256) / tiles;
    p = p < kSkMaxPieces ? p : kSkMaxPieces;
    const int64_t by_k = one_row ? K / 256 : (K / 256) / 3;
    p = p < by_k ? p : by_k;
    return p > 1 ? (int)p : 1;
}

bool form_shape_ok(int form, int64_t M, int64_t N, int64_t K)
{
    if (check_mmq_shape(M, N, K) != QPG_OK) return false;
    if (form == 2) return prep_shape_ok(N, K);
    if (form == 3) return exp_shape_ok(N, K) && form_tiles(3, M, N, K) < kMaxDim;
    return form >= 0 && form <= 1;
}

int mmq_sk_checked(int form, const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                   size_t ws_bytes, hipStream_t st)
{
    if (!w || !xq || !y) return QPG_EINVAL;
    if (!form_shape_ok(form, M, N, K)) return QPG_EINVAL;
    const int P = sk_pieces(form, M, N, K);
    if (P > 1) {
        if (!ws || ws_bytes < (size_t)P * (size_t)M * (size_t)N * 4) return QPG_EINVAL;
        if (!aligned(ws, 16)) return QPG_EALIGN;
    }
    const uintptr_t wa = form == 1 ? 2 : 16;
    if (!aligned(w, wa) || !aligned(xq, 16) || !aligned(y, 4)) return QPG_EALIGN;
    const int rc = check_device();
    if (rc != QPG_OK) return rc;
    float* out = P > 1 ? static_cast<float*>(ws) : y;
    hipError_t e;
    switch (form) {
    case 0: e = qpg_launch_mmq_q4K(w, xq, out, nullptr, M, N, K, P, st); break;
    case 1: e = qpg_launch_mmq_q6K(w, xq, out, nullptr, M, N, K, P, st); break;
    case 2: e = qpg_launch_mmq_q6K_prep(w, xq, out, nullptr, M, N, K, P, st); break;
    default: e = qpg_launch_mmq_q6K_exp(w, xq, out, nullptr, M, N, K, P, st); break;
    }
    if (e == hipSuccess && P > 1) e = qpg_launch_splitk_reduce(static_cast<const float*>(ws), y, M * N, P, st);
    return status_of(e);
}

}  // namespace

extern "C" {

size_t qpg_mmq_sk_bytes(int64_t M, int64_t N, int64_t K, int form)
{
    if (form < 0 || form > 3 || !form_shape_ok(form, M, N, K)) return 0;
    const int P = sk_pieces(form, M, N, K);
    return P > 1 ? (size_t)P * (size_t)M * (size_t)N * 4 : 0;
}

int mmq_q4K_q8_sk(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                  size_t ws_bytes, qpg_stream_t stream)
{
    return mmq_sk_checked(0, w, xq, y, M, N, K, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_q8_sk(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                  size_t ws_bytes, qpg_stream_t stream)
{
    return mmq_sk_checked(1, w, xq, y, M, N, K, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_prep_q8_sk(const void* wp, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                       size_t ws_bytes, qpg_stream_t stream)
{
    return mmq_sk_checked(2, wp, xq, y, M, N, K, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_exp_q8_sk(const void* we, const void* xq, float* y, int64_t M, int64_t N, int64_t K, void* ws,
                      size_t ws_bytes, qpg_stream_t stream)
{
    return mmq_sk_checked(3, we, xq, y, M, N, K, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

size_t qpg_q6K_exp_bytes(int64_t N, int64_t K)
{
    if (!exp_shape_ok(N, K)) return 0;
    return (size_t)(((N + kExpTile - 1) / kExpTile) * (K / 256) * kExpSb);
}

int q6K_expand(const void* w, void* we, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!w || !we) return QPG_EINVAL;
    if (!exp_shape_ok(N, K)) return QPG_EINVAL;
    if (!aligned(we, 16)) return QPG_EALIGN;
    const int rc = check_device();
    if (rc != QPG_OK) return rc;
    return status_of(qpg_launch_q6K_expand(w, we, N, K, reinterpret_cast<hipStream_t>(stream)));
}

int mmq_q6K_exp_q8(const void* we, const void* xq, float* y, int64_t M, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!y) return QPG_EINVAL;
    return mmq_exp_checked(we, xq, y, nullptr, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_exp_csums(const void* we, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                      qpg_stream_t stream)
{
    if (!s) return QPG_EINVAL;
    return mmq_exp_checked(we, xq, nullptr, s, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

size_t qpg_q6K_prep_bytes(int64_t N, int64_t K)
{
    if (!prep_shape_ok(N, K)) return 0;
    return (size_t)(((N + kPrepTile - 1) / kPrepTile) * (K / 256) * kPrepSb);
}

int q6K_prepare(const void* w, void* wp, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!w || !wp) return QPG_EINVAL;
    if (!prep_shape_ok(N, K)) return QPG_EINVAL;
    if (!aligned(w, 4) || !aligned(wp, 16)) return QPG_EALIGN;
    const int rc = check_device();
    if (rc != QPG_OK) return rc;
    return status_of(qpg_launch_q6K_prepare(w, wp, N, K, reinterpret_cast<hipStream_t>(stream)));
}

int mmq_q6K_prep_q8(const void* wp, const void* xq, float* y, int64_t M, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!y) return QPG_EINVAL;
    return mmq_prep_checked(wp, xq, y, nullptr, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_prep_isums(const void* wp, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                       qpg_stream_t stream)
{
    if (!s) return QPG_EINVAL;
    return mmq_prep_checked(wp, xq, nullptr, s, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

const char* qpg_strerror(int status)
{
    switch (status) {
    case QPG_OK: return "ok";
    case QPG_EINVAL: return "invalid argument (null pointer or unsupported shape)";
    case QPG_EALIGN: return "pointer alignment requirement violated";
    case QPG_EHIP: return "HIP runtime error while enqueuing";
    case QPG_EDEVICE: return "current device is not gfx950 (MI355X) or cannot be queried";
    case QPG_ESCRATCH: return "q8_1 activations larger than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
    }
}

size_t qpg_q8_1_bytes(int64_t M, int64_t K)
{
    if (M < 1 || K < 32 || K % 32 != 0 || M >= kMaxDim || K >= kMaxDim) return 0;
    return (size_t)(M * K + 4 * M * (K / 32));
}

int quantize_q8_1(const float* x, void* xq, int64_t M, int64_t K, qpg_stream_t stream)
{
    return quantize_checked(x, xq, M, K, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q4K_q8(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!y) return QPG_EINVAL;
    return mmq_checked(false, w, xq, y, nullptr, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_q8(const void* w, const void* xq, float* y, int64_t M, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!y) return QPG_EINVAL;
    return mmq_checked(true, w, xq, y, nullptr, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q4K_isums(const void* w, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                  qpg_stream_t stream)
{
    if (!s) return QPG_EINVAL;
    return mmq_checked(false, w, xq, nullptr, s, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

int mmq_q6K_isums(const void* w, const void* xq, int32_t* s, int64_t M, int64_t N, int64_t K,
                  qpg_stream_t stream)
{
    if (!s) return QPG_EINVAL;
    return mmq_checked(true, w, xq, nullptr, s, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

static int mmq_f32(bool q6, const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K, void* xq_ws,
                   qpg_stream_t stream)
{
    if (!w || !x || !y || !xq_ws) return QPG_EINVAL;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int rc = check_mmq_shape(M, N, K);
    if (rc != QPG_OK) return rc;
    if (!aligned(x, 16) || !aligned(xq_ws, 16) || !aligned(w, q6 ? 2 : 16) || !aligned(y, 4)) return QPG_EALIGN;
    rc = quantize_checked(x, xq_ws, M, K, s);
    if (rc != QPG_OK) return rc;
    return mmq_checked(q6, w, xq_ws, y, nullptr, M, N, K, s);
}

int mmq_q4K(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K, void* xq_ws,
            qpg_stream_t stream)
{
    return mmq_f32(false, w, x, y, M, N, K, xq_ws, stream);
}

int mmq_q6K(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K, void* xq_ws,
            qpg_stream_t stream)
{
    return mmq_f32(true, w, x, y, M, N, K, xq_ws, stream);
}

int mmq_q4K_noalloc(const void* w, const float* x, float* y, int64_t M, int64_t N, int64_t K, qpg_stream_t stream)
{
    if (!w || !x || !y) return QPG_EINVAL;
    int rc = check_mmq_shape(M, N, K);
    if (rc != QPG_OK) return rc;
    if (qpg_q8_1_bytes(M, K) > (size_t)QPG_NOALLOC_SCRATCH_BYTES) return QPG_ESCRATCH;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 4)) return QPG_EALIGN;
    rc = check_device();
    if (rc != QPG_OK) return rc;
    void* xq = nullptr;
    rc = scratch_of_current_device(&xq);
    if (rc != QPG_OK) return rc;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    rc = quantize_checked(x, xq, M, K, s);
    if (rc != QPG_OK) return rc;
    return mmq_checked(false, w, xq, y, nullptr, M, N, K, s);
}

}  // extern "C"
