// Test stubs of the kernel launchers and device-side size helpers that the
// C-ABI validation layer (api.cpp) calls, so that layer can be built on the
// host alone with AddressSanitizer and UndefinedBehaviorSanitizer.  A stub
// never reads or writes a buffer (the driver passes fake device addresses);
// it counts the launch and reports success.  The size helpers return simple
// stand-ins of the library's values: the driver only needs them to be
// consistent between the *_workspace_bytes calls and the calls they size.
#include <hip/hip_runtime.h>

#include "qt_internal.h"

int qt_stub_launches = 0;

namespace qt {

static hipError_t counted() {
    ++qt_stub_launches;
    return hipSuccess;
}

hipError_t launch_quantize_g64(const float*, int64_t, int64_t, const float*, int, int, bool, int,
                               const GridTable&, float*, int8_t*, uint8_t*, hipStream_t) {
    return counted();
}
hipError_t launch_pack_i3(const int8_t*, int64_t, int64_t, uint8_t*, hipStream_t) { return counted(); }
hipError_t launch_pack_i4(const int8_t*, int64_t, int64_t, uint8_t*, hipStream_t) { return counted(); }
hipError_t launch_gemv_batch(const uint8_t*, const float*, int64_t, int64_t, const void*, bool,
                             int64_t, float*, hipStream_t, int) {
    return counted();
}
hipError_t launch_gemv_grouped(const uint8_t*, const float*, int32_t, int64_t, int64_t,
                               const float*, int64_t, const int32_t*, const int32_t*, int32_t,
                               float*, hipStream_t, int) {
    return counted();
}
hipError_t launch_gemm_mfma(const uint8_t*, const float*, int64_t, int64_t, const uint16_t*,
                            int64_t, float*, hipStream_t) {
    return counted();
}
int64_t hessian_full_rows(int64_t I) { return (I + 127) / 128 * 128; }
int64_t hessian_full_tokens(int64_t T) { return (T + 63) / 64 * 64; }
hipError_t launch_hessian_full(const void*, bool, int64_t, int64_t, float*, int, void*,
                               hipStream_t) {
    return counted();
}
size_t gptq_factor_workspace(int64_t n) { return (size_t)n * (size_t)n * 8; }
hipError_t launch_gptq_factor(const float*, int64_t, double, float*, int32_t*, void*,
                              hipStream_t) {
    return counted();
}
size_t gptq_workspace(int64_t O, int64_t I) { return (size_t)O * (size_t)I * 8; }
hipError_t launch_gptq_i3(const float*, int64_t, int64_t, const float*, float*, int8_t*, void*,
                          hipStream_t) {
    return counted();
}
int64_t proxy_pad(int64_t n) { return (n + 127) / 128 * 128; }
size_t gptq_proxy_workspace(int64_t O, int64_t I) {
    return (size_t)proxy_pad(2 * O) * (size_t)proxy_pad(I) * 4;
}
hipError_t launch_gptq_proxy(const float*, const uint8_t*, const float*, int64_t, int64_t,
                             const float*, double*, void*, hipStream_t) {
    return counted();
}
size_t moe_layer_workspace(int64_t T, int64_t k, int64_t E, int64_t D, int64_t F) {
    return (size_t)(T * k) * (size_t)(2 * F + D) * 4 + (size_t)(E + 1) * 64;
}
hipError_t launch_moe_layer(const float*, int64_t, int64_t, int64_t, const float*, int32_t,
                            int32_t, const uint8_t*, const float*, int, const uint8_t*,
                            const float*, int, const uint8_t*, const float*, int, float*, void*,
                            hipStream_t) {
    return counted();
}
int hessian_slabs(int64_t T, int64_t) { return T <= 128 ? 1 : (int)((T + 127) / 128 > 128 ? 128 : (T + 127) / 128); }
// a fixed fake device address: the no-allocation entry point only passes it on
void* hessian_scratch_ptr() { return reinterpret_cast<void*>(uintptr_t(0x7E0000000000ULL)); }
hipError_t launch_hessian_diag(const void*, bool, int64_t, int64_t, float*, int, float*,
                               hipStream_t) {
    return counted();
}

}  // namespace qt
