// Per-group scale search, code emission and packing for int3-g64 and grouped
// int4.
//
// Method: the "int3-g64 (fmt=5)" pull request page ("Why this format" item 1:
// a 3-bit group-64 absmax quantizer; "Design", Layout bullet: 24 bytes per
// group, codes in [-4,3] stored as v+4) and the NeUQI accuracy page (first
// paragraph: candidate scales searched on a grid, weighted by activation
// importance).  Grouped int4 (the grouped-int4 format of the int3-g64 page,
// "Design" and the OLMoE per-projection table) is the same quantizer with
// b = 4: base absmax/8, codes in [-8,7], stored as nibbles of v+8.  Every f32 operation of the objective is a separately rounded
// operation (this file is compiled without floating-point contraction), and
// the 64 slot errors are summed by halving, so the chosen candidate is a
// bit-exact function of the inputs.
#include "qt_internal.h"

namespace qt {
namespace {

constexpr int kLanesPerGroup = 16;  // a quarter wave owns one group
constexpr int kQuantBlock = 256;    // 16 groups per block

// The b-bit symmetric group quantizer: base = absmax * 2^-(b-1), codes v in
// [-2^(b-1), 2^(b-1) - 1].  With base normal, 2^(b-1) * base == absmax exactly.
template <int BITS>
struct Range {
    static_assert(BITS == 3 || BITS == 4, "int3 or int4 codes");
    static constexpr float kHalf = (float)(1 << (BITS - 1));  // 4 or 8
    static constexpr float kLo = -kHalf;
    static constexpr float kHi = kHalf - 1.0f;
    static constexpr float kBase = 1.0f / kHalf;  // exact power of two
};

// q = clamp(rne(fl(w / s)), lo, hi), 0 when s == 0, where fl(w / s) is the
// correctly rounded f32 quotient.
template <int BITS>
__device__ __forceinline__ float code_of(float w, float s) {
    if (s == 0.0f) return 0.0f;
    float q = __builtin_rintf(w / s);
    return fminf(fmaxf(q, Range<BITS>::kLo), Range<BITS>::kHi);
}

// A single candidate (the plain group quantizer, s = base * f0): no
// objective to evaluate, so the group's 16 lanes take 4 consecutive inputs
// each (16-byte loads), share the absmax through DPP steps inside their
// 16-lane row (the maximum does not depend on the order) and store their four
// codes as one word.  VEC: W rows allow 16-byte loads and code rows 4-byte
// stores (I % 4 == 0, W 16-byte and codes 4-byte aligned).
template <int BITS, bool VEC>
__global__ __launch_bounds__(kQuantBlock) void quantize_rtn_kernel(
    const float* __restrict__ W, int64_t n_groups, int32_t I, int32_t G, float f0,
    float* __restrict__ scales, int8_t* __restrict__ codes, uint8_t* __restrict__ grid_idx) {
    const int l = threadIdx.x & (kLanesPerGroup - 1);
    const int64_t grp = (int64_t)blockIdx.x * (kQuantBlock / kLanesPerGroup) +
                        (threadIdx.x / kLanesPerGroup);
    if (grp >= n_groups) return;  // a whole 16-lane row leaves together
    const int64_t o = grp / G;
    const int32_t g = (int32_t)(grp - o * G);
    const int32_t c0 = g * kGroup;
    const int32_t n = min(kGroup, I - c0);
    const float* w = W + o * (int64_t)I + c0;
    float wv[4];
    if (VEC && n == kGroup) {
        const float4 v = *reinterpret_cast<const float4*>(w + 4 * l);
        wv[0] = v.x;
        wv[1] = v.y;
        wv[2] = v.z;
        wv[3] = v.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * l + e;
            wv[e] = j < n ? w[j] : 0.0f;
        }
    }
    float amax = fmaxf(fmaxf(fabsf(wv[0]), fabsf(wv[1])), fmaxf(fabsf(wv[2]), fabsf(wv[3])));
    // quad_perm [1,0,3,2], [2,3,0,1], then row_ror 4 and 8: every lane of the
    // row ends with the row's maximum
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1,
                                                                  0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E,
                                                                  0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x124,
                                                                  0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x128,
                                                                  0xF, 0xF, false)));
    const float s = amax * Range<BITS>::kBase * f0;
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        word |= ((uint32_t)(int)code_of<BITS>(wv[e], s) & 0xFFu) << (8 * e);
    int8_t* cd = codes + o * (int64_t)I + c0 + 4 * l;
    if (VEC && n == kGroup) {
        *reinterpret_cast<uint32_t*>(cd) = word;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * l + e < n) cd[e] = (int8_t)(word >> (8 * e));
    }
    if (l == 0) {
        scales[grp] = s;
        if (grid_idx) grid_idx[grp] = 0;
    }
}

// ---------------------------------------------------------------- search
// With more than one candidate the work is 64 candidates x 64 slots of
// arithmetic per group, so one lane owns a whole group: the halving sum is
// then lane-local (63 adds per candidate instead of a cross-lane reduction),
// the per-candidate set-up (scale, reciprocal, comparison) is paid once per
// 64 slots, and a wave's 64 lanes take 64 rows of the same group column, so
// the importance weights d are the same for the whole wave (scalar registers).
constexpr int kSearchRows = 64;  // one wave per block, one row per lane

enum QuotientMode { kReciprocal, kDivision };

// Halving sum of the 64 slot errors of one candidate with scale s.  In
// kReciprocal mode the codes come from y = fl(w * r), r = rcp(s), and *dev
// receives the largest |y - rint(y)| for the exactness check; kDivision uses
// the correctly rounded quotient (0 when s == 0).  Why the check suffices:
// r = v_rcp_f32(s) is within 1 ulp of 1/s, so y and the correctly rounded
// fl(w/s) differ by at most 2^-22 |w/s|; the per-candidate margin leaves
// twice that bound (for the largest |w/s| the group can hold) between y and
// every half-integer, so wherever |y - rint(y)| < margin, fl(w/s) rounds to
// the same integer as y.  Groups outside the margin, or whose scales leave
// [2^-100, 2^100], are decided with the division.
template <bool WEIGHTED, int MODE, int BITS>
__device__ __forceinline__ float group_error(const float (&w)[kGroup], const float (&dj)[kGroup],
                                             float s, float r, float* dev) {
    float a[32];
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        float e2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int jj = j + 32 * h;
            float q;
            if (MODE == kReciprocal) {
                const float y = w[jj] * r;
                q = __builtin_rintf(y);
                mx = fmaxf(mx, fabsf(y - q));
            } else {
                q = s == 0.0f ? 0.0f : __builtin_rintf(w[jj] / s);
            }
            const float qc = __builtin_amdgcn_fmed3f(q, Range<BITS>::kLo, Range<BITS>::kHi);
            const float t = s * qc;
            const float rr = w[jj] - t;
            const float r2 = rr * rr;
            e2[h] = WEIGHTED ? dj[jj] * r2 : r2;  // padding slots: w = 0, d = 0
        }
        a[j] = e2[0] + e2[1];  // m = 32
    }
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1)
#pragma unroll
        for (int j = 0; j < m; ++j) a[j] = a[j] + a[j + m];
    if (MODE == kReciprocal) *dev = mx;
    return a[0];
}

// Exactness margin for a factor f computed on the device (the second stage of
// the signed search): the host's bound 2^(b-1)/f (1 + 2^-20) with extra slack
// that covers the f32 rounding of this formula; a smaller margin only sends
// more candidates to the division.
template <int BITS>
__device__ __forceinline__ float device_margin(float f) {
    const float bound = Range<BITS>::kHalf / f * 1.001f;
    return bound < 0x1p20f ? 0.5f - bound * 0x1p-21f : 0.0f;
}

// SIGNED: the two-stage signed search of the NeUQI page.  Stage 1 takes every
// factor of the grid with both signs (k ascending, + before -); stage 2 takes
// n2 points of [f_{k-1}, f_{k+1}] around the stage-1 winner k with its sign,
// formed in double exactly as the grid itself; the final choice is the strict
// minimum over [stage-1 winner, stage-2 points], so ties keep the earlier one.
template <bool WEIGHTED, bool SIGNED, int BITS>
__global__ __launch_bounds__(kSearchRows) void search_g64_kernel(
    const float* __restrict__ W, int64_t O, int32_t I, int32_t G,
    const float* __restrict__ d, int32_t ncand, int32_t n2, GridTable tab, int vec,
    float* __restrict__ scales, int8_t* __restrict__ codes, uint8_t* __restrict__ grid_idx) {
    // consecutive blocks walk the group columns of one 64-row slab
    const int64_t rb = blockIdx.x / G;
    const int32_t g = (int32_t)(blockIdx.x - rb * G);
    const int64_t o = rb * kSearchRows + threadIdx.x;
    if (o >= O) return;  // no cross-lane operations below
    const int32_t c0 = g * kGroup;
    const int32_t n = min(kGroup, I - c0);
    const float* wp = W + o * (int64_t)I + c0;

    float w[kGroup], dj[kGroup];
    if (vec) {  // I % 4 == 0 and W 16-byte aligned: n is a multiple of 4
#pragma unroll
        for (int c = 0; c < kGroup / 4; ++c) {
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (4 * c < n) v = reinterpret_cast<const float4*>(wp)[c];
            w[4 * c + 0] = v.x;
            w[4 * c + 1] = v.y;
            w[4 * c + 2] = v.z;
            w[4 * c + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) w[j] = j < n ? wp[j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) dj[j] = (WEIGHTED && j < n) ? d[c0 + j] : 0.0f;

    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) amax = fmaxf(amax, fabsf(w[j]));
    const float base = amax * Range<BITS>::kBase;
    // base normal: 2^(b-1) * base == amax exactly, so every |w| <= 2^(b-1) *
    // base; and
    // s = fl(base * f) is monotone in f, so checking the smallest and the
    // largest factor covers every candidate
    const bool group_ok = base >= 0x1p-125f && base * tab.fmin >= 0x1p-100f &&
                          base * tab.fmax <= 0x1p100f;

    // objective of one candidate scale (reciprocal quotients, division where
    // the exactness margin does not hold)
    auto error_of = [&](float s, float margin) {
        const float r = __builtin_amdgcn_rcpf(s);
        float dev;
        float a = group_error<WEIGHTED, kReciprocal, BITS>(w, dj, s, r, &dev);
        if (!(group_ok && dev < margin))  // rare: some quotient near a half-integer
            a = group_error<WEIGHTED, kDivision, BITS>(w, dj, s, r, nullptr);
        return a;
    };
    float best_e = 0.0f, best_s = 0.0f, best_margin = 0.0f;
    int best_k = 0;
    for (int k = 0; k < ncand; ++k) {
        const float s = base * tab.f[k];
        const float margin = tab.margin[k];
        const float a = error_of(s, margin);
        if (k == 0 || a < best_e) {  // strict: the lowest k wins ties
            best_e = a;
            best_k = k;
            best_s = s;
            best_margin = margin;
        }
        if constexpr (SIGNED) {
            const float an = error_of(-s, margin);
            if (an < best_e) {
                best_e = an;
                best_k = k;
                best_s = -s;
                best_margin = margin;
            }
        }
    }
    if constexpr (SIGNED) {
        if (n2 > 0) {
            // the winner's neighbours on the grid (per lane: a global read of
            // the kernel-argument table)
            const float fa = tab.f[best_k > 0 ? best_k - 1 : 0];
            const float fb = tab.f[best_k < ncand - 1 ? best_k + 1 : ncand - 1];
            const double step = ((double)fb - (double)fa) / (double)(n2 - 1);
            const bool neg = __builtin_signbit(best_s);
            for (int j = 0; j < n2; ++j) {
                const float f = j == n2 - 1 ? fb : (float)((double)fa + (double)j * step);
                const float mag = base * f;
                const float s = neg ? -mag : mag;
                const float margin = device_margin<BITS>(f);
                const float a = error_of(s, margin);
                if (a < best_e) {
                    best_e = a;
                    best_s = s;
                    best_margin = margin;
                }
            }
        }
    }

    // codes of the chosen scale, by the same exactness rule per slot
    const float s = best_s;
    const float r = __builtin_amdgcn_rcpf(s);
    uint32_t packed4[kGroup / 4];
#pragma unroll
    for (int c = 0; c < kGroup / 4; ++c) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = 4 * c + b;
            const float y = w[j] * r;
            float q = __builtin_rintf(y);
            if (!(group_ok && fabsf(y - q) < best_margin))
                q = s == 0.0f ? 0.0f : __builtin_rintf(w[j] / s);
            const int v = (int)__builtin_amdgcn_fmed3f(q, Range<BITS>::kLo, Range<BITS>::kHi);
            word |= ((uint32_t)v & 0xFFu) << (8 * b);
        }
        packed4[c] = word;
    }
    int8_t* cp = codes + o * (int64_t)I + c0;
    if (vec == 2 && n == kGroup) {  // I % 16 == 0, W and codes 16-byte aligned
#pragma unroll
        for (int c = 0; c < kGroup / 16; ++c)
            reinterpret_cast<uint4*>(cp)[c] = make_uint4(packed4[4 * c], packed4[4 * c + 1],
                                                         packed4[4 * c + 2], packed4[4 * c + 3]);
    } else {
        for (int j = 0; j < n; ++j) cp[j] = (int8_t)(packed4[j >> 2] >> (8 * (j & 3)));
    }
    const int64_t grp = o * G + g;
    scales[grp] = s;
    if (!SIGNED && grid_idx) grid_idx[grp] = (uint8_t)best_k;
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
    // Byte-parallel: word q holds slots 4q..4q+3, which are exactly low byte
    // q (two bits each) and high bits 4q..4q+3.
    uint32_t lb[16];  // low byte q in bits 0..7 (higher bits are not used)
    uint32_t hi[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        // u = (v + 4) mod 8 in every byte: flipping bit 2 of the low three
        // bits of v (no carry crosses a byte)
        const uint32_t u4 = (c[q] & 0x07070707u) ^ 0x04040404u;
        // low two bits of byte b to bits 2b..2b+1 of byte 0
        const uint32_t t = u4 & 0x03030303u;
        const uint32_t x = t | (t >> 6);  // bytes 0 and 2: two slots each
        lb[q] = x | (x >> 12);
        // bit 2 of byte b to bit b of a nibble: the product's terms land on
        // distinct bits (no carries), bits 21..24 hold the four
        const uint32_t h = (u4 >> 2) & 0x01010101u;
        const uint32_t nib = ((h * 0x00204081u) >> 21) & 0xFu;
        hi[q >> 3] |= nib << (4 * (q & 7));
    }
    uint32_t lo[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // bytes 0 of lb[4w .. 4w+3] side by side
        const uint32_t p01 = __builtin_amdgcn_perm(lb[4 * w + 1], lb[4 * w], 0x0C0C0400u);
        const uint32_t p23 = __builtin_amdgcn_perm(lb[4 * w + 3], lb[4 * w + 2], 0x04000C0Cu);
        lo[w] = p01 | p23;
    }
    uint2* dst = reinterpret_cast<uint2*>(packed + grp * kGroupBytes);
    dst[0] = make_uint2(lo[0], lo[1]);
    dst[1] = make_uint2(lo[2], lo[3]);
    dst[2] = make_uint2(hi[0], hi[1]);
}

// One thread per group: 64 codes in, 32 packed bytes out (two 16-byte
// stores; groups start on 32-byte boundaries).  Slot j goes to the low nibble
// of byte j/2 when j is even, to the high nibble when j is odd, as u = v + 8;
// padding holds u = 8.
__global__ __launch_bounds__(256) void pack_i4_kernel(const int8_t* __restrict__ codes,
                                                       int64_t n_groups, int32_t I, int32_t G,
                                                       int vec16, uint8_t* __restrict__ packed) {
    const int64_t grp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (grp >= n_groups) return;
    const int64_t o = grp / G;
    const int32_t g = (int32_t)(grp - o * G);
    const int32_t c0 = g * kGroup;
    const int32_t n = min(kGroup, I - c0);
    const int8_t* src = codes + o * (int64_t)I + c0;

    uint32_t c[16];  // 64 codes, 4 per word, little-endian bytes; padding v = 0
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
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
        uint32_t h[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            // u = (v + 8) mod 16 in every byte: flipping bit 3 of the low four
            // bits of v; then bytes (u0, u1, u2, u3) -> half-word u0 | u1 << 4
            // | u2 << 8 | u3 << 12
            const uint32_t u = (c[q + k] & 0x0F0F0F0Fu) ^ 0x08080808u;
            const uint32_t t = u | (u >> 4);  // byte 0: u0 | u1 << 4, byte 2: u2 | u3 << 4
            h[k] = (t & 0xFFu) | ((t >> 8) & 0xFF00u);
        }
        out[q >> 1] = h[0] | (h[1] << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(packed + grp * kGroupBytesI4);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

template <int BITS>
hipError_t quantize_bits(const float* W, int64_t O, int64_t I, const float* d, int ncand,
                         int n2, bool signed_search, const GridTable& tab, float* scales,
                         int8_t* codes, uint8_t* grid_idx, hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    if (ncand > 1 || signed_search) {
        // lane-per-group search: blocks = G * ceil(O / 64)
        const bool w16 = (reinterpret_cast<uintptr_t>(W) & 15) == 0;
        const bool c16 = (reinterpret_cast<uintptr_t>(codes) & 15) == 0;
        const int vec = (w16 && I % 4 == 0) ? ((c16 && I % 16 == 0) ? 2 : 1) : 0;
        const int64_t blocks = G * ((O + kSearchRows - 1) / kSearchRows);
        if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define QT_SEARCH(WT, SG)                                                                \
    hipLaunchKernelGGL((search_g64_kernel<WT, SG, BITS>), dim3((unsigned)blocks),          \
                       dim3(kSearchRows), 0, s, W, O, (int32_t)I, (int32_t)G, d, ncand, n2, \
                       tab, vec, scales, codes, grid_idx)
        if (signed_search) {
            if constexpr (BITS == 3) {
                if (d)
                    QT_SEARCH(true, true);
                else
                    QT_SEARCH(false, true);
            } else {
                return hipErrorInvalidValue;  // the signed search is int3 only
            }
        } else {
            if (d)
                QT_SEARCH(true, false);
            else
                QT_SEARCH(false, false);
        }
#undef QT_SEARCH
        return hipGetLastError();
    }
    const int64_t n_groups = O * G;
    const int64_t per_block = kQuantBlock / kLanesPerGroup;
    const int64_t blocks = (n_groups + per_block - 1) / per_block;
    if (ncand == 1) {  // the plain quantizer: d does not change the choice
        const bool vec = (I % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(codes) & 3) == 0);
        if (vec)
            hipLaunchKernelGGL((quantize_rtn_kernel<BITS, true>), dim3((unsigned)blocks),
                               dim3(kQuantBlock), 0, s, W, n_groups, (int32_t)I, (int32_t)G,
                               tab.f[0], scales, codes, grid_idx);
        else
            hipLaunchKernelGGL((quantize_rtn_kernel<BITS, false>), dim3((unsigned)blocks),
                               dim3(kQuantBlock), 0, s, W, n_groups, (int32_t)I, (int32_t)G,
                               tab.f[0], scales, codes, grid_idx);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;  // ncand >= 1
}

}  // namespace

hipError_t launch_quantize_g64(const float* W, int64_t O, int64_t I, const float* d,
                               int ncand, int n2, bool signed_search, int bits,
                               const GridTable& tab, float* scales, int8_t* codes,
                               uint8_t* grid_idx, hipStream_t s) {
    if (bits == 3)
        return quantize_bits<3>(W, O, I, d, ncand, n2, signed_search, tab, scales, codes,
                                grid_idx, s);
    if (bits == 4)
        return quantize_bits<4>(W, O, I, d, ncand, n2, signed_search, tab, scales, codes,
                                grid_idx, s);
    return hipErrorInvalidValue;
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

hipError_t launch_pack_i4(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed,
                          hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    const int64_t n_groups = O * G;
    const int vec16 = ((reinterpret_cast<uintptr_t>(codes) & 15) == 0) && (I % 16 == 0);
    const int64_t blocks = (n_groups + 255) / 256;
    hipLaunchKernelGGL(pack_i4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes,
                       n_groups, (int32_t)I, (int32_t)G, vec16, packed);
    return hipGetLastError();
}

}  // namespace qt
