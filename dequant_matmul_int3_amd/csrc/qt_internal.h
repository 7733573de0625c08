// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Arguments here are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qt {

constexpr int kGroup = 64;       // inputs per group
constexpr int kGroupBytes = 24;  // int3: 16 B low plane + 8 B high plane
constexpr int kGroupBytesI4 = 32;  // int4: 64 nibbles
constexpr int kMaxGrid = 256;    // largest candidate grid of the scale search

// Candidate factors of the scale search, passed by value as a kernel argument.
// Candidate scale factors and, per factor, the rounding margin the search
// kernel uses to accept a reciprocal-based quotient without a division.
struct GridTable {
    float f[kMaxGrid];
    float margin[kMaxGrid];
    float fmin, fmax;
};

// ncand candidates of tab; signed_search: the two-stage signed search with n2
// second-stage points (0: stage 1 only; int3 only).  bits: 3 or 4.
hipError_t launch_quantize_g64(const float* W, int64_t O, int64_t I, const float* d,
                               int ncand, int n2, bool signed_search, int bits,
                               const GridTable& tab, float* scales, int8_t* codes,
                               uint8_t* grid_idx, hipStream_t s);

hipError_t launch_pack_i3(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed,
                          hipStream_t s);
hipError_t launch_pack_i4(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed,
                          hipStream_t s);

// Dequantize-multiply of `ntok` input rows against one O x I matrix, exact-f32
// path.  X rows are f32 (bf16 == false) or bf16 bit patterns (bf16 == true).
// bits: 3 (24-byte int3 groups) or 4 (32-byte int4 groups).
hipError_t launch_gemv_batch(const uint8_t* packed, const float* scales, int64_t O,
                             int64_t I, const void* X, bool bf16, int64_t ntok,
                             float* Y, hipStream_t s, int bits = 3);

// bits: 3 (int3-g64 experts) or 4 (grouped int4 experts).
hipError_t launch_gemv_grouped(const uint8_t* packed, const float* scales, int32_t E,
                               int64_t O, int64_t I, const float* X, int64_t n_x_rows,
                               const int32_t* pair_row, const int32_t* expert_offsets,
                               int32_t P, float* Y, hipStream_t s, int bits = 3);

// bf16 MFMA path, B >= 16.
hipError_t launch_gemm_mfma(const uint8_t* packed, const float* scales, int64_t O,
                            int64_t I, const uint16_t* X, int64_t B, float* Y,
                            hipStream_t s);

// Full Hessian, GPTQ factor, sweep and proxy (syrk.hip, factor.hip, gptq.hip).
int64_t hessian_full_rows(int64_t I);
int64_t hessian_full_tokens(int64_t T);
hipError_t launch_hessian_full(const void* X, bool bf16, int64_t T, int64_t I, float* H,
                               int accumulate, void* workspace, hipStream_t s);
hipError_t launch_rowdot_nt(const float* A, int64_t Mp, const float* B, int64_t Np, int64_t Kp,
                            float* part, hipStream_t s);
size_t gptq_factor_workspace(int64_t n);
hipError_t launch_gptq_factor(const float* H, int64_t n, double damp, float* U, int32_t* info,
                              void* workspace, hipStream_t s);
size_t gptq_workspace(int64_t O, int64_t I);
hipError_t launch_gptq_i3(const float* W, int64_t O, int64_t I, const float* U, float* scales,
                          int8_t* codes, void* workspace, hipStream_t s);
int64_t proxy_pad(int64_t n);
size_t gptq_proxy_workspace(int64_t O, int64_t I);
hipError_t launch_gptq_proxy(const float* W, const uint8_t* packed, const float* scales,
                             int64_t O, int64_t I, const float* H, double* terms,
                             void* workspace, hipStream_t s);

// MoE expert layer (moe.hip): routing, gate/up, SwiGLU, down and combine launches.
size_t moe_layer_workspace(int64_t T, int64_t k, int64_t E, int64_t D, int64_t F);
hipError_t launch_moe_layer(const float* X, int64_t T, int64_t D, int64_t F,
                            const float* logits, int32_t E, int32_t k, const uint8_t* gp,
                            const float* gs, int gbits, const uint8_t* up, const float* us,
                            int ubits, const uint8_t* dp, const float* ds, int dbits, float* out,
                            void* workspace, hipStream_t s);

int hessian_slabs(int64_t T, int64_t I);
// Bytes of the built-in scratch of qt_hessian_diag_noalloc, and its device
// address on the current device (NULL on failure).
constexpr size_t kHessianScratchBytes = size_t(16) << 20;
void* hessian_scratch_ptr();
hipError_t launch_hessian_diag(const void* X, bool bf16, int64_t T, int64_t I, float* d,
                               int accumulate, float* workspace, hipStream_t s);

}  // namespace qt
