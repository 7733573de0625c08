// Importance weights for the scale search: the diagonal of H = sum_t X^T X,
// d[j] = sum_t X[t,j]^2 (the tt-stack issue page, pipeline table step 1:
// H per linear input accumulated over the calibration tokens in fp32 on the
// device; only its diagonal enters the per-group weighted objective).
//
// Streaming column reduction, bound by HBM reads of X.  Stage 1: the grid is
// (column tiles) x (token slabs); a thread owns VEC adjacent columns (one
// 16-byte load per token row) and sums the squares of its slab's rows in f32.
// Stage 2 adds the slab partials along a fixed tree.  No atomics: the result
// is independent of scheduling.
#include <algorithm>
#include <atomic>

#include "qt_internal.h"

// Scratch of the allocation-free entry point (slab partials): a file-scope
// device array, so that callers that cannot allocate still get a fixed-order
// reduction.  Each device holds its own copy until the process ends; calls
// on one device share it.
static __device__ __align__(256) float scratch[qt::kHessianScratchBytes / sizeof(float)];

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kHesThreads = 256;
constexpr int kTokPerSlab = 128;  // rows of X per slab
constexpr int kMaxSlabs = 128;
constexpr int kUnroll = 8;        // row loads in flight per thread

template <int VEC, bool BF16>
__device__ __forceinline__ void load_row(const void* X, int64_t idx, float (&v)[VEC]) {
    if (BF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(X) + idx;
        if (VEC == 8) {
            const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = __uint_as_float(w[e] << 16);
                v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = __uint_as_float((uint32_t)p[e] << 16);
        }
    } else {
        const float* p = reinterpret_cast<const float*>(X) + idx;
        if (VEC == 4) {
            const f32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
            v[0] = q.x;
            v[1] = q.y;
            v[2] = q.z;
            v[3] = q.w;
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = p[e];
        }
    }
}

// out[s*I + j] (or d when there is one slab) for the columns of this thread.
template <int VEC, bool BF16>
__global__ __launch_bounds__(kHesThreads) void hessian_partial_kernel(
    const void* __restrict__ X, int64_t T, int64_t I, int64_t rows_per_slab,
    float* __restrict__ out, int direct, int accumulate) {
    const int64_t c = ((int64_t)blockIdx.x * kHesThreads + threadIdx.x) * VEC;
    if (c >= I) return;
    const int64_t s = blockIdx.y;
    const int64_t t0 = s * rows_per_slab;
    const int64_t t1 = std::min<int64_t>(T, t0 + rows_per_slab);
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    int64_t t = t0;
    for (; t + kUnroll <= t1; t += kUnroll) {
        float v[kUnroll][VEC];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) load_row<VEC, BF16>(X, (t + u) * I + c, v[u]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(v[u][e], v[u][e], acc[e]);
    }
    for (; t < t1; ++t) {
        float v[VEC];
        load_row<VEC, BF16>(X, t * I + c, v);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = __builtin_fmaf(v[e], v[e], acc[e]);
    }
    if (direct) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) out[c + e] = accumulate ? out[c + e] + acc[e] : acc[e];
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) out[s * I + c + e] = acc[e];
    }
}

// Stage 2: a block owns kCombCols columns; thread (column c, part q) adds
// the slab partials q, q + kCombParts, ... in slab order, then part 0 adds the
// kCombParts sums in part order.  The summation tree is fixed, so the result
// does not depend on scheduling.
constexpr int kCombCols = 32;
constexpr int kCombParts = kHesThreads / kCombCols;  // 8

__global__ __launch_bounds__(kHesThreads) void hessian_combine_kernel(
    const float* __restrict__ part, int64_t I, int slabs, float* __restrict__ d,
    int accumulate) {
    __shared__ float sums[kCombParts][kCombCols];
    const int c = threadIdx.x % kCombCols, q = threadIdx.x / kCombCols;
    const int64_t j = (int64_t)blockIdx.x * kCombCols + c;
    const int64_t jc = j < I ? j : I - 1;  // columns past I: read a valid one, unused
    float total = 0.0f;
    for (int s = q; s < slabs; s += kCombParts) total += part[(int64_t)s * I + jc];
    sums[q][c] = total;
    __syncthreads();
    if (q == 0 && j < I) {
        float t = sums[0][c];
#pragma unroll
        for (int k = 1; k < kCombParts; ++k) t += sums[k][c];
        d[j] = accumulate ? d[j] + t : t;
    }
}

template <int VEC, bool BF16>
hipError_t run(const void* X, int64_t T, int64_t I, float* d, int accumulate, float* ws,
               int slabs, hipStream_t st) {
    const int64_t rows = (T + slabs - 1) / slabs;
    const int64_t threads = (I + VEC - 1) / VEC;
    const dim3 grid((unsigned)((threads + kHesThreads - 1) / kHesThreads), (unsigned)slabs);
    const int direct = slabs == 1;
    hipLaunchKernelGGL((hessian_partial_kernel<VEC, BF16>), grid, dim3(kHesThreads), 0, st, X,
                       T, I, rows, direct ? d : ws, direct, accumulate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL(hessian_combine_kernel, dim3((unsigned)((I + kCombCols - 1) / kCombCols)),
                       dim3(kHesThreads), 0, st, ws, I, slabs, d, accumulate);
    return hipGetLastError();
}

}  // namespace

int hessian_slabs(int64_t T, int64_t I) {
    (void)I;
    const int64_t s = (T + kTokPerSlab - 1) / kTokPerSlab;
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, kMaxSlabs));
}

hipError_t launch_hessian_diag(const void* X, bool bf16, int64_t T, int64_t I, float* d,
                               int accumulate, float* workspace, hipStream_t s) {
    const int slabs = hessian_slabs(T, I);
    const bool aligned = (reinterpret_cast<uintptr_t>(X) & 15) == 0;
    if (bf16) {
        if (aligned && I % 8 == 0) return run<8, true>(X, T, I, d, accumulate, workspace, slabs, s);
        return run<1, true>(X, T, I, d, accumulate, workspace, slabs, s);
    }
    if (aligned && I % 4 == 0) return run<4, false>(X, T, I, d, accumulate, workspace, slabs, s);
    return run<1, false>(X, T, I, d, accumulate, workspace, slabs, s);
}

// Device address of `scratch` on the current device, taken once per device
// (the array's name in host code is only a stand-in, not a device address).
// NULL if the runtime cannot give it.
void* hessian_scratch_ptr() {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    addr[dev].store(q, std::memory_order_release);  // two racing threads store the same address
    return q;
}

}  // namespace qt
