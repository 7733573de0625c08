// Drives every entry point of include/qt.h through the host-side validation
// layer (api.cpp built with AddressSanitizer and UndefinedBehaviorSanitizer,
// the kernel launchers replaced by launch_stubs.cpp).  Buffers are fake,
// far-apart device addresses that nothing dereferences.  Each call checks
// the returned status; valid calls reach a stub and return QT_OK.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <limits>

#include "qt.h"

extern int qt_stub_launches;

namespace {

int failures = 0;

#define EXPECT(call, want)                                                               \
    do {                                                                                 \
        const int got_ = (int)(call);                                                    \
        if (got_ != (int)(want)) {                                                       \
            std::printf("FAIL %s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, \
                        got_, (int)(want));                                              \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

template <typename T = void>
T* at(uint64_t base, uint64_t off = 0) {
    return reinterpret_cast<T*>(static_cast<uintptr_t>(base + off));
}

const uint64_t A = 0x7F0000000000ULL, B = 0x7F1000000000ULL, C = 0x7F2000000000ULL,
               D = 0x7F3000000000ULL, E = 0x7F4000000000ULL, F = 0x7F5000000000ULL,
               W = 0x7F6000000000ULL, H = 0x7F7000000000ULL, K = 0x7F8000000000ULL,
               L = 0x7F9000000000ULL, M = 0x7FA000000000ULL, N = 0x7FB000000000ULL;
const int64_t BIG = std::numeric_limits<int64_t>::max();

void sizes() {
    EXPECT(qt_groups(0), 0);
    EXPECT(qt_groups(-5), 0);
    EXPECT(qt_groups(7200), 113);
    EXPECT(qt_groups(BIG) > 0, 1);
    EXPECT(qt_packed_bytes(2048, 7168), 5505024);
    EXPECT(qt_packed_bytes(BIG, BIG), 0);
    EXPECT(qt_packed_bytes(1LL << 62, 1LL << 20), 0);
    EXPECT(qt_packed_bytes_i4(BIG, 64), 0);
    for (int s = -1; s <= 10; ++s) EXPECT(qt_status_str((qt_status)s) != nullptr, 1);
    EXPECT(qt_hessian_workspace_bytes(BIG, BIG), 0);
    EXPECT(qt_hessian_workspace_bytes(-1, 64), 0);
    EXPECT(qt_hessian_scratch_bytes() > 0, 1);
}

void hessian() {
    EXPECT(qt_hessian_diag(nullptr, QT_F32, 8, 64, at<float>(B), 0, nullptr, 0, nullptr), QT_ERR_NULL);
    EXPECT(qt_hessian_diag(at(A), (qt_dtype)7, 8, 64, at<float>(B), 0, nullptr, 0, nullptr), QT_ERR_DTYPE);
    EXPECT(qt_hessian_diag(at(A), QT_F32, BIG, BIG, at<float>(B), 0, nullptr, 0, nullptr), QT_ERR_SHAPE);
    EXPECT(qt_hessian_diag(at(A), QT_F32, BIG / 2, 64, at<float>(B), 0, nullptr, 0, nullptr), QT_ERR_SHAPE);
    EXPECT(qt_hessian_diag(at(A), QT_F32, 8, 64, at<float>(B), 2, nullptr, 0, nullptr), QT_ERR_ARG);
    EXPECT(qt_hessian_diag(at(A, 2), QT_F32, 8, 64, at<float>(B), 0, nullptr, 0, nullptr), QT_ERR_ALIGN);
    EXPECT(qt_hessian_diag(at(A, 2), QT_BF16, 8, 64, at<float>(B), 0, nullptr, 0, nullptr), QT_OK);
    EXPECT(qt_hessian_diag(at(A), QT_F32, 8, 64, at<float>(A, 64), 0, nullptr, 0, nullptr), QT_ERR_ALIAS);
    const size_t need = qt_hessian_workspace_bytes(8192, 17408);
    EXPECT(need > 0, 1);
    EXPECT(qt_hessian_diag(at(A), QT_F32, 8192, 17408, at<float>(B), 0, nullptr, 0, nullptr), QT_ERR_WORKSPACE);
    EXPECT(qt_hessian_diag(at(A), QT_F32, 8192, 17408, at<float>(B), 1, at(C), need, nullptr), QT_OK);
    EXPECT(qt_hessian_diag(at(A), QT_F32, 8192, 17408, at<float>(B), 0, at(A, 4), need, nullptr), QT_ERR_ALIAS);
    EXPECT(qt_hessian_diag_noalloc(at(A), QT_F32, 8192, 17408, at<float>(B), 0, nullptr), QT_OK);
    EXPECT(qt_hessian_diag_noalloc(at(A), QT_F32, 8192, 1 << 20, at<float>(B), 0, nullptr), QT_ERR_SCRATCH);
    EXPECT(qt_hessian_diag_noalloc(at(A), QT_F32, 8, 64, at<float>(B), 0, nullptr), QT_OK);
    EXPECT(qt_hessian_diag_noalloc(nullptr, QT_F32, 8, 64, at<float>(B), 0, nullptr), QT_ERR_NULL);
}

void quantize() {
    const float nan = std::nanf("");
    EXPECT(qt_quantize_g64(nullptr, 4, 64, nullptr, 0, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_NULL);
    EXPECT(qt_quantize_g64(at<float>(A), 0, 64, nullptr, 0, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_SHAPE);
    EXPECT(qt_quantize_g64(at<float>(A), BIG, BIG, nullptr, 0, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_SHAPE);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 1, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 300, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 64, nan, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 64, 1.0f, 0.5f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 64, -1.0f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64(at<float>(A, 2), 4, 64, nullptr, 64, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_ERR_ALIGN);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 64, 0.5f, 1.0f, at<float>(A, 8), at<int8_t>(C), nullptr, nullptr), QT_ERR_ALIAS);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, at<float>(D), 64, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), at<uint8_t>(E), nullptr), QT_OK);
    EXPECT(qt_quantize_g64(at<float>(A), 4, 64, nullptr, 0, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_OK);
    EXPECT(qt_quantize_g64(at<float>(A), 3, 7200, nullptr, 256, 0.25f, 4.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_OK);
    EXPECT(qt_quantize_g64_signed(at<float>(A), 4, 64, nullptr, 64, 32, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr), QT_OK);
    EXPECT(qt_quantize_g64_signed(at<float>(A), 4, 64, nullptr, 64, 1, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64_signed(at<float>(A), 4, 64, nullptr, 0, 0, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr), QT_ERR_ARG);
    EXPECT(qt_quantize_g64_i4(at<float>(A), 4, 64, nullptr, 64, 0.5f, 1.0f, at<float>(B), at<int8_t>(C), nullptr, nullptr), QT_OK);
}

void pack_and_multiply() {
    EXPECT(qt_pack_i3(at<int8_t>(A), 2, 64, at<uint8_t>(B), nullptr), QT_OK);
    EXPECT(qt_pack_i3(at<int8_t>(A), 2, 64, at<uint8_t>(B, 4), nullptr), QT_OK);
    EXPECT(qt_pack_i3(at<int8_t>(A), 2, 64, at<uint8_t>(B, 2), nullptr), QT_ERR_ALIGN);
    EXPECT(qt_pack_i3(at<int8_t>(A), 2, 64, at<uint8_t>(A, 16), nullptr), QT_ERR_ALIAS);
    EXPECT(qt_pack_i4(at<int8_t>(A), 2, 64, at<uint8_t>(B, 4), nullptr), QT_ERR_ALIGN);
    EXPECT(qt_pack_i4(at<int8_t>(A), 2, 64, at<uint8_t>(B), nullptr), QT_OK);

    EXPECT(qt_matvec_i3(at<uint8_t>(A, 4), at<float>(B), 4, 64, at<float>(C), at<float>(D), nullptr), QT_OK);
    EXPECT(qt_matvec_i3(at<uint8_t>(A), at<float>(B), 4, 64, at<float>(C), at<float>(C, 4), nullptr), QT_ERR_ALIAS);
    EXPECT(qt_matvec_i4(at<uint8_t>(A, 4), at<float>(B), 4, 64, at<float>(C), at<float>(D), nullptr), QT_ERR_ALIGN);
    EXPECT(qt_matvec_i4(at<uint8_t>(A), at<float>(B), 4, 64, at<float>(C), at<float>(D), nullptr), QT_OK);

    for (int64_t b : {1, 15, 16, 512}) {
        EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 18432, 7168, at(C, 2), QT_BF16, b, at<float>(D), nullptr), QT_OK);
        EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 18432, 7168, at(C), QT_F32, b, at<float>(D), nullptr), QT_OK);
        EXPECT(qt_matmul_i4(at<uint8_t>(A), at<float>(B), 2048, 7168, at(C, 2), QT_BF16, b, at<float>(D), nullptr), QT_OK);
    }
    EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 4, 64, at(C), (qt_dtype)9, 2, at<float>(D), nullptr), QT_ERR_DTYPE);
    EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 4, 64, at(C), QT_F32, BIG, at<float>(D), nullptr), QT_ERR_SHAPE);
    EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 1LL << 40, 1LL << 20, at(C), QT_F32, 1 << 22, at<float>(D), nullptr), QT_ERR_SHAPE);  // B*O*4 overflows
    EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 4, 64, at(C, 1), QT_BF16, 32, at<float>(D), nullptr), QT_ERR_ALIGN);
    EXPECT(qt_matmul_i3(at<uint8_t>(A), at<float>(B), 4, 64, at(C), QT_BF16, 32, at<float>(C, 64), nullptr), QT_ERR_ALIAS);

    const int32_t E_ = 128;
    EXPECT(qt_matvec_i3_grouped(at<uint8_t>(A, 4), at<float>(B), E_, 2048, 7168, at<float>(C), 32, at<int32_t>(D), at<int32_t>(E), 256, at<float>(F), nullptr), QT_OK);
    EXPECT(qt_matvec_i3_grouped(at<uint8_t>(A), at<float>(B), 0, 2048, 7168, at<float>(C), 32, nullptr, at<int32_t>(E), 256, at<float>(F), nullptr), QT_ERR_SHAPE);
    EXPECT(qt_matvec_i3_grouped(at<uint8_t>(A), at<float>(B), E_, 2048, 7168, at<float>(C), 32, nullptr, at<int32_t>(E), 256, at<float>(F), nullptr), QT_ERR_SHAPE);
    EXPECT(qt_matvec_i3_grouped(at<uint8_t>(A), at<float>(B), E_, 2048, 7168, at<float>(C), 32, at<int32_t>(D, 2), at<int32_t>(E), 256, at<float>(F), nullptr), QT_ERR_ALIGN);
    EXPECT(qt_matvec_i3_grouped(at<uint8_t>(A), at<float>(B), E_, 2048, 7168, at<float>(C), 32, at<int32_t>(D), at<int32_t>(E), 256, at<float>(B, 64), nullptr), QT_ERR_ALIAS);
    EXPECT(qt_matvec_i4_grouped(at<uint8_t>(A), at<float>(B), E_, 2048, 7168, at<float>(C), 32, at<int32_t>(D), at<int32_t>(E), 256, at<float>(F), nullptr), QT_OK);
    EXPECT(qt_matvec_i4_grouped(at<uint8_t>(A, 4), at<float>(B), E_, 2048, 7168, at<float>(C), 32, at<int32_t>(D), at<int32_t>(E), 256, at<float>(F), nullptr), QT_ERR_ALIGN);
}

void gptq_and_moe() {
    const size_t hw = qt_hessian_full_workspace_bytes(8192, 17408, QT_BF16);
    EXPECT(hw > 0, 1);
    EXPECT(qt_hessian_full(at(A), QT_BF16, 8192, 17408, at<float>(H), 0, at(K), hw, nullptr), QT_OK);
    EXPECT(qt_hessian_full(at(A), QT_BF16, 8192, 17408, at<float>(H), 0, at(K), hw - 1, nullptr), QT_ERR_WORKSPACE);
    EXPECT(qt_hessian_full(nullptr, QT_BF16, 8192, 17408, at<float>(H), 0, at(K), hw, nullptr), QT_ERR_NULL);
    EXPECT(qt_hessian_full_workspace_bytes(BIG, BIG, QT_F32), 0);
    const size_t fw = qt_gptq_factor_workspace_bytes(17408);
    EXPECT(qt_gptq_factor(at<float>(H), 17408, 0.01, at<float>(L), at<int32_t>(M), at(K), fw, nullptr), QT_OK);
    EXPECT(qt_gptq_factor(at<float>(H), 17408, -1.0, at<float>(L), at<int32_t>(M), at(K), fw, nullptr), QT_ERR_ARG);
    EXPECT(qt_gptq_factor(at<float>(H), 17408, std::nan(""), at<float>(L), at<int32_t>(M), at(K), fw, nullptr), QT_ERR_ARG);
    const size_t gw = qt_gptq_workspace_bytes(5120, 17408);
    EXPECT(qt_gptq_i3(at<float>(W), 5120, 17408, at<float>(L), at<float>(B), at<int8_t>(C), at(K), gw, nullptr), QT_OK);
    EXPECT(qt_gptq_i3(at<float>(W), 5120, 17408, at<float>(L), at<float>(B), at<int8_t>(W, 64), at(K), gw, nullptr), QT_ERR_ALIAS);
    const size_t pw = qt_gptq_proxy_workspace_bytes(5120, 17408);
    EXPECT(qt_gptq_proxy(at<float>(W), at<uint8_t>(A), at<float>(B), 5120, 17408, at<float>(H), at<double>(N), at(K), pw, nullptr), QT_OK);
    EXPECT(qt_gptq_proxy(at<float>(W), at<uint8_t>(A), at<float>(B), 5120, 17408, at<float>(H), at<double>(N, 4), at(K), pw, nullptr), QT_ERR_ALIGN);
    const size_t mw = qt_moe_layer_workspace_bytes(32, 8, 128, 7168, 2048);
    EXPECT(mw > 0, 1);
    EXPECT(qt_moe_layer(at<float>(C), 32, 7168, 2048, at<float>(D), 128, 8, at<uint8_t>(A),
                        at<float>(B), 3, at<uint8_t>(E), at<float>(F), 3, at<uint8_t>(H),
                        at<float>(L), 3, at<float>(M), at(K), mw, nullptr), QT_OK);
    EXPECT(qt_moe_layer(at<float>(C), 32, 7168, 2048, at<float>(D), 128, 8, at<uint8_t>(A),
                        at<float>(B), 5, at<uint8_t>(E), at<float>(F), 3, at<uint8_t>(H),
                        at<float>(L), 3, at<float>(M), at(K), mw, nullptr), QT_ERR_ARG);
    EXPECT(qt_moe_layer(at<float>(C), 32, 7168, 2048, at<float>(D), 128, 0, at<uint8_t>(A),
                        at<float>(B), 3, at<uint8_t>(E), at<float>(F), 3, at<uint8_t>(H),
                        at<float>(L), 3, at<float>(M), at(K), mw, nullptr) != QT_OK, 1);
    EXPECT(qt_moe_layer_workspace_bytes(BIG, 8, 128, 7168, 2048), 0);
}

}  // namespace

int main() {
    sizes();
    hessian();
    quantize();
    pack_and_multiply();
    gptq_and_moe();
    std::printf("%d stub launches, %d failures\n", qt_stub_launches, failures);
    return failures == 0 ? 0 : 1;
}
