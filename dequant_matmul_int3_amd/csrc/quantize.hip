// Per-group scale search, code emission and bit-plane packing for int3-g64.
//
// Method: the "int3-g64 (fmt=5)" pull request page ("Why this format" item 1:
// a 3-bit group-64 absmax quantizer; "Design", Layout bullet: 24 bytes per
// group, codes in [-4,3] stored as v+4) and the NeUQI accuracy page (first
// paragraph: candidate scales searched on a grid, weighted by activation
// importance).  Every f32 operation of the objective is a separately rounded
// operation (this file is compiled without floating-point contraction), and
// the 64 slot errors are summed by halving, so the chosen candidate is a
// bit-exact function of the inputs.
#include "qt_internal.h"

namespace qt {
namespace {

constexpr int kLanesPerGroup = 16;  // a quarter wave owns one group
constexpr int kQuantBlock = 256;    // 16 groups per block

// q = clamp(rne(fl(w / s)), -4, 3), 0 when s == 0, where fl(w / s) is the
// correctly rounded f32 quotient.
__device__ __forceinline__ float code_of(float w, float s) {
    if (s == 0.0f) return 0.0f;
    float q = __builtin_rintf(w / s);
    return fminf(fmaxf(q, -4.0f), 3.0f);
}

// The same code without a division on the common path.  With r = rcp(s)
// (v_rcp_f32: within 1 ulp of 1/s) and y = fl(w * r), |y - w/s| and
// |fl(w/s) - w/s| together stay below 2.4e-7 * |w/s|, i.e. below
// |y| * 2^-21 for every finite y.  When y is farther than that from every
// half-integer, fl(w/s) lies strictly on the same side of each half-integer
// as y, so rint(y) == rint(fl(w/s)).  Otherwise (and for s outside
// [2^-100, 2^100], or |y| >= 2^22) the correctly rounded division decides.
__device__ __forceinline__ float code_fast(float w, float s, float r, bool s_ok) {
    const float y = w * r;
    const float q = __builtin_rintf(y);
    const float d = fabsf(y - q);  // exact for |y| < 2^22: distance to the nearest integer
    const float margin = 0.5f - fabsf(y) * 0x1p-21f;
    float c = q;
    if (!(s_ok && fabsf(y) < 0x1p22f && d < margin)) c = __builtin_rintf(w / s);
    return fminf(fmaxf(c, -4.0f), 3.0f);
}

// One halving step of the slot errors: lane l (l < m) of a 16-lane row adds
// the partial sum of lane l + m (row_shl:m moves lane l+m's value to lane l).
template <int M>
__device__ __forceinline__ float add_from_lane_plus(float a) {
    const int v = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0x100 + M, 0xF, 0xF, true);
    return a + __builtin_bit_cast(float, v);
}

// Lane l of a quarter wave holds slots l, l+16, l+32, l+48 of its group, so
// the first two halving steps (m = 32, 16) are lane-local and the remaining
// four (m = 8, 4, 2, 1) read the partner lane l + m through DPP.
__global__ __launch_bounds__(kQuantBlock) void quantize_g64_kernel(
    const float* __restrict__ W, int64_t n_groups, int32_t I, int32_t G,
    const float* __restrict__ d, int32_t ncand, GridTable tab,
    float* __restrict__ scales, int8_t* __restrict__ codes,
    uint8_t* __restrict__ grid_idx) {
    const int l = threadIdx.x & (kLanesPerGroup - 1);
    const int64_t grp = (int64_t)blockIdx.x * (kQuantBlock / kLanesPerGroup) +
                        (threadIdx.x / kLanesPerGroup);
    // grp is uniform over the 16 lanes of a group (one DPP row), so a whole
    // row leaves together and the cross-lane reads below see only live lanes
    // of the same group.
    if (grp >= n_groups) return;
    const int64_t o = grp / G;
    const int32_t g = (int32_t)(grp - o * G);
    const int32_t c0 = g * kGroup;
    const int32_t n = min(kGroup, I - c0);
    const float* w = W + o * (int64_t)I + c0;

    float wv[4], dv[4];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = l + 16 * e;
        const bool ok = j < n;
        wv[e] = ok ? w[j] : 0.0f;
        dv[e] = ok ? (d ? d[c0 + j] : 1.0f) : 0.0f;
        amax = fmaxf(amax, fabsf(wv[e]));
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kLanesPerGroup));
    const float base = amax * 0.25f;

    float best_e = 0.0f;
    int best_k = 0;
#pragma unroll 4
    for (int k = 0; k < ncand; ++k) {
        const float s = base * tab.f[k];
        const float r = __builtin_amdgcn_rcpf(s);
        const bool s_ok = s >= 0x1p-100f && s <= 0x1p100f;
        float e4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float q = s == 0.0f ? 0.0f : code_fast(wv[e], s, r, s_ok);
            const float t = s * q;
            const float rr = wv[e] - t;
            const float r2 = rr * rr;
            e4[e] = dv[e] * r2;  // padding slots: dv = 0 and rr = 0 give +0
        }
        // m = 32: slots j and j+32 are e4[0] + e4[2] and e4[1] + e4[3];
        // m = 16: slot l gets slot l+16.
        const float a32_lo = e4[0] + e4[2];
        const float a32_hi = e4[1] + e4[3];
        float a = a32_lo + a32_hi;
        // m = 8, 4, 2, 1: slot l (l < m) gets slot l + m, held by lane l + m
        a = add_from_lane_plus<8>(a);
        a = add_from_lane_plus<4>(a);
        a = add_from_lane_plus<2>(a);
        a = add_from_lane_plus<1>(a);
        if (k == 0 || a < best_e) {  // strict: the lowest k wins ties
            best_e = a;
            best_k = k;
        }
    }
    // lane 0 of the quarter wave holds the halving sum and the choice
    best_k = __shfl(best_k, 0, kLanesPerGroup);
    const float s = base * tab.f[best_k];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = l + 16 * e;
        if (j < n) codes[o * (int64_t)I + c0 + j] = (int8_t)(int)code_of(wv[e], s);
    }
    if (l == 0) {
        scales[grp] = s;
        if (grid_idx) grid_idx[grp] = (uint8_t)best_k;
    }
}

// One thread per group: 64 codes in, 24 packed bytes out (three 8-byte
// stores; groups start on 8-byte boundaries).  Slot 4b+i goes to bits 2i..2i+1
// of low byte b, slot 8c+i to bit i of high byte c; padding holds u = 4.
__global__ __launch_bounds__(256) void pack_i3_kernel(const int8_t* __restrict__ codes,
                                                       int64_t n_groups, int32_t I, int32_t G,
                                                       int vec16, uint8_t* __restrict__ packed) {
    const int64_t grp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (grp >= n_groups) return;
    const int64_t o = grp / G;
    const int32_t g = (int32_t)(grp - o * G);
    const int32_t c0 = g * kGroup;
    const int32_t n = min(kGroup, I - c0);
    const int8_t* src = codes + o * (int64_t)I + c0;

    uint32_t c[16];  // 64 codes, 4 per word, little-endian bytes
    if (vec16 && n == kGroup) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = s4[q];
            c[4 * q + 0] = v.x;
            c[4 * q + 1] = v.y;
            c[4 * q + 2] = v.z;
            c[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            uint32_t wv = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int j = 4 * q + b;
                const uint32_t byte = j < n ? (uint8_t)src[j] : 0u;
                wv |= byte << (8 * b);
            }
            c[q] = wv;
        }
    }
    uint32_t lo[4] = {0, 0, 0, 0};
    uint32_t hi[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        // u = (v + 4) mod 8 in every byte: flipping bit 2 of the low three
        // bits of v (no carry crosses a byte)
        const uint32_t u4 = (c[q] & 0x07070707u) ^ 0x04040404u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t u = (u4 >> (8 * b)) & 7u;
            const int j = 4 * q + b;  // slot index in the group
            lo[j >> 4] |= (u & 3u) << (2 * (j & 15));
            hi[j >> 5] |= (u >> 2) << (j & 31);
        }
    }
    uint2* dst = reinterpret_cast<uint2*>(packed + grp * kGroupBytes);
    dst[0] = make_uint2(lo[0], lo[1]);
    dst[1] = make_uint2(lo[2], lo[3]);
    dst[2] = make_uint2(hi[0], hi[1]);
}

}  // namespace

hipError_t launch_quantize_g64(const float* W, int64_t O, int64_t I, const float* d,
                               int ncand, const GridTable& tab, float* scales,
                               int8_t* codes, uint8_t* grid_idx, hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    const int64_t n_groups = O * G;
    const int64_t per_block = kQuantBlock / kLanesPerGroup;
    const int64_t blocks = (n_groups + per_block - 1) / per_block;
    hipLaunchKernelGGL(quantize_g64_kernel, dim3((unsigned)blocks), dim3(kQuantBlock), 0, s, W,
                       n_groups, (int32_t)I, (int32_t)G, d, ncand, tab, scales, codes,
                       grid_idx);
    return hipGetLastError();
}

hipError_t launch_pack_i3(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed,
                          hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    const int64_t n_groups = O * G;
    const int vec16 = ((reinterpret_cast<uintptr_t>(codes) & 15) == 0) && (I % 16 == 0);
    const int64_t blocks = (n_groups + 255) / 256;
    hipLaunchKernelGGL(pack_i3_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes,
                       n_groups, (int32_t)I, (int32_t)G, vec16, packed);
    return hipGetLastError();
}

}  // namespace qt
