// Host-sanitizer driver of the C ABI (tests/test_sanitize.py builds it together with the
// library sources under -Xarch_host -fsanitize=address / undefined): every entry point with
// arguments its validation must reject -- null pointers, bad shapes, misaligned pointers,
// an undersized split-K workspace, a q8_1 buffer beyond the allocation-free scratch -- all of
// which return before the device is touched. With argument "nodevice" (a machine without a
// GPU) valid arguments are passed too and must report QPG_EDEVICE. No kernel is launched.
#include <cstdio>
#include <cstring>

#include "../../include/qpg.h"
#include "../../include/qpg_calib.h"

#define CHECK(cond)                                                                    \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);   \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

int main(int argc, char** argv)
{
    const bool nodevice = argc > 1 && std::strcmp(argv[1], "nodevice") == 0;
    void* A16 = reinterpret_cast<void*>(1 << 20);           // never dereferenced
    void* A8 = reinterpret_cast<void*>((1 << 20) + 8);
    void* A2 = reinterpret_cast<void*>((1 << 20) + 2);
    void* A1 = reinterpret_cast<void*>((1 << 20) + 1);
    float* F16 = static_cast<float*>(A16);
    float* F8 = static_cast<float*>(A8);
    for (int c = -6; c <= 1; ++c) CHECK(qpg_strerror(c) != nullptr);
    CHECK(qpg_q8_1_bytes(512, 4096) == 512u * 4096u + 4u * 512u * 128u && qpg_q8_1_bytes(0, 256) == 0);
    CHECK(qpg_q6K_prep_bytes(0, 256) == 0 && qpg_q6K_exp_bytes(64, 300) == 0 && qpg_mmq_sk_bytes(1, 1, 256, 9) == 0);

    CHECK(quantize_q8_1(nullptr, A16, 4, 256, nullptr) == QPG_EINVAL);
    CHECK(quantize_q8_1(F16, A16, 4, 48, nullptr) == QPG_EINVAL);
    CHECK(quantize_q8_1(F8, A16, 4, 256, nullptr) == QPG_EALIGN);
    CHECK(mmq_q4K(A16, F16, F16, 64, 256, 256, nullptr, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K(A16, F8, F16, 64, 256, 256, A16, nullptr) == QPG_EALIGN);
    CHECK(mmq_q4K_q8(A16, A16, F16, 0, 256, 256, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_q8(A1, A16, F16, 64, 256, 256, nullptr) == QPG_EALIGN);
    CHECK(mmq_q4K_isums(A16, A16, nullptr, 64, 256, 256, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_isums(A16, A16, static_cast<int32_t*>(A16), 64, 256, 288, nullptr) == QPG_EINVAL);
    CHECK(q6K_prepare(A2, A16, 128, 256, nullptr) == QPG_EALIGN);
    CHECK(mmq_q6K_prep_q8(A16, A16, F16, 64, 256, 1 << 24, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_prep_isums(A8, A16, static_cast<int32_t*>(A16), 64, 256, 256, nullptr) == QPG_EALIGN);
    CHECK(q6K_expand(A16, nullptr, 64, 256, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_exp_q8(A16, A16, F16, 64, 256, 1 << 24, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_exp_csums(A16, A16, static_cast<int32_t*>(A2), 64, 256, 256, nullptr) == QPG_EALIGN);
    const size_t need = qpg_mmq_sk_bytes(512, 512, 4096, 0), need6 = qpg_mmq_sk_bytes(512, 512, 4096, 1);
    CHECK(need == 4u * 512u * 512u * 4u && need6 == 5u * 512u * 512u * 4u);
    CHECK(mmq_q4K_q8_sk(A16, A16, F16, 512, 512, 4096, A16, need - 4, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_q8_sk(A16, A16, F16, 512, 512, 4096, A8, need6, nullptr) == QPG_EALIGN);
    CHECK(mmq_q6K_prep_q8_sk(A16, A16, F16, 512, 512, 288, A16, need6, nullptr) == QPG_EINVAL);
    CHECK(mmq_q6K_exp_q8_sk(nullptr, A16, F16, 512, 512, 4096, A16, need6, nullptr) == QPG_EINVAL);
    CHECK(mmq_q4K_noalloc(A16, F16, F16, 2711, 256, 11008, nullptr) == QPG_ESCRATCH);
    CHECK(mmq_q4K_noalloc(A8, F16, F16, 64, 256, 256, nullptr) == QPG_EALIGN);
    CHECK(qpg_calib_mfma_i8(0, 10, static_cast<uint64_t*>(A16), nullptr) == -1);
    CHECK(qpg_calib_step(8, 3, 10, static_cast<uint64_t*>(A16), nullptr) == -1);
    CHECK(qpg_probe_mfma(0, A8, A16, A16, A16, nullptr) == -2);
    CHECK(qpg_probe_lds_dma(4, A16, 1024, nullptr, static_cast<uint32_t*>(A16), nullptr) == -1);
    if (nodevice) {
        CHECK(quantize_q8_1(F16, A16, 64, 256, nullptr) == QPG_EDEVICE);
        CHECK(mmq_q4K_q8(A16, A16, F16, 64, 256, 256, nullptr) == QPG_EDEVICE);
        CHECK(mmq_q6K_q8(A2, A16, F16, 64, 256, 256, nullptr) == QPG_EDEVICE);   // 2-byte q6_K blocks
        CHECK(mmq_q4K_noalloc(A16, F16, F16, 64, 256, 256, nullptr) == QPG_EDEVICE);
        CHECK(mmq_q6K_exp_q8_sk(A16, A16, F16, 64, 256, 4096, A16, 8u * 64u * 256u * 4u, nullptr) == QPG_EDEVICE);
        CHECK(qpg_calib_step_blocks(3) == 0);
    }
    std::printf("abi driver: ok\n");
    return 0;
}
