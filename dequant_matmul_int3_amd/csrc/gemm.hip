// int3-g64 dequantize-and-multiply for batches of bf16 activations on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Y[t,o] = sum_g s[o,g] * sum_{j<64} v[o,64g+j] * X[t,64g+j]
//
// The int3 codes v in [-4,3] are exact in bf16, so each group's 64-term dot
// product is formed by the matrix cores with exact products and f32
// accumulation, and is then multiplied by the f32 group scale on the vector
// ALUs and added into an f32 accumulator: the per-group scale accumulation of
// the matmul_i3 kernel ("int3-g64 (fmt=5)" pull request page, "Design", Kernel
// bullet), with bf16 inputs.
//
// Tiling: a block of 4 waves computes a 128 (tokens) x 128 (output rows) tile
// and walks the input dimension one 64-wide group at a time.  The activation
// tile of the next group is fetched into registers while the current one is
// consumed from LDS (double-buffered, one barrier per group).  Each wave owns a
// 64 x 64 sub-tile = 2 x 2 MFMA tiles of 32 x 32.  The B operand is built in
// registers straight from the packed planes: a lane loads the 24 bytes of its
// output row's group and turns 8 codes per k-step into 8 bf16 values through
// byte-permute table lookups (v_perm_b32), no LDS round trip.
//
// k order inside a group: k-step s (0..3) of 16 inputs takes codes
// 16s .. 16s+15; lanes 0..31 supply codes 16s..16s+7 and lanes 32..63 codes
// 16s+8..16s+15 of A and B alike, so every product pairs the same input.
#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int BM = 128;          // tokens per block tile
constexpr int BN = 128;          // output rows per block tile
constexpr int kThreads = 256;    // 4 waves
constexpr int XROW = kGroup + 8; // bf16 per LDS row (16 bytes of padding)

// 4 codes (one u = v+4 per byte) -> their bf16 values as [lo0 hi0 lo1 hi1],
// [lo2 hi2 lo3 hi3].  Table bytes: bf16(v) for v = -4..3 is c080 c040 c000
// bf80 0000 3f80 4000 4040.
__device__ __forceinline__ void codes_to_bf16(uint32_t U, uint32_t& d0, uint32_t& d1) {
    const uint32_t hi = __builtin_amdgcn_perm(0x40403F00u, 0xBFC0C0C0u, U);
    const uint32_t lo = __builtin_amdgcn_perm(0x40008000u, 0x80004080u, U);
    d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// 8 consecutive codes -> bf16x8.  lo16: their 2-bit low fields (code e at bits
// 2e), hi8: their high bits (code e at bit e).
__device__ __forceinline__ bf16x8_t eight_codes(uint32_t lo16, uint32_t hi8) {
    uint32_t r[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        uint32_t f = (lo16 >> (8 * half)) & 0xFFu;  // four 2-bit fields
        f = (f | (f << 12)) & 0x000F000Fu;
        f = (f | (f << 6)) & 0x03030303u;             // field e -> byte e
        const uint32_t h = (hi8 >> (4 * half)) & 0xFu;
        // bit e of h -> bit 8e+2 (the four partial products never overlap)
        const uint32_t hb = (h * 0x00810204u) & 0x04040404u;
        codes_to_bf16(f | hb, r[2 * half], r[2 * half + 1]);
    }
    u32x4_t v = {r[0], r[1], r[2], r[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_i3_mfma_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int64_t I,
    int64_t G, const uint16_t* __restrict__ X, int64_t B, float* __restrict__ Y) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * XROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // token half of the block tile
    const int wn = wave >> 1;  // output-row half
    const int h = lane >> 5;   // which 8 codes of a k-step
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;

    // this lane's two output rows (one per 32-wide n tile)
    int64_t orow[2];
    bool orow_ok[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        orow[nt] = n0 + wn * 64 + nt * 32 + (lane & 31);
        orow_ok[nt] = orow[nt] < O;
    }

    // activation tile loader: 128 rows x 64 bf16 = 1024 chunks of 8
    auto load_x = [&](int64_t g, u32x4_t (&buf)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3;
            const int col = (c & 7) * 8;
            const int64_t t = m0 + row;
            const int64_t k = g * kGroup + col;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (t < B) {
                const uint16_t* src = X + t * I + k;
                if (VEC) {
                    if (k < I) v = *reinterpret_cast<const u32x4_t*>(src);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t a = (k + 2 * e < I) ? src[2 * e] : 0u;
                        const uint32_t b = (k + 2 * e + 1 < I) ? src[2 * e + 1] : 0u;
                        w[e] = a | (b << 16);
                    }
                    v = u32x4_t{w[0], w[1], w[2], w[3]};
                }
            }
            buf[i] = v;
        }
    };
    auto store_x = [&](int b, const u32x4_t (&buf)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3;
            const int col = (c & 7) * 8;
            *reinterpret_cast<u32x4_t*>(&xs[b][row * XROW + col]) = buf[i];
        }
    };
    struct WGroup {
        uint2 a, b, c;
        float s;
    };
    auto load_w = [&](int64_t g, WGroup (&w)[2]) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            if (orow_ok[nt]) {
                const int64_t gi = orow[nt] * G + g;
                const uint2* p = reinterpret_cast<const uint2*>(packed + gi * kGroupBytes);
                w[nt].a = p[0];
                w[nt].b = p[1];
                w[nt].c = p[2];
                w[nt].s = scales[gi];
            } else {
                // rows past O: any codes, zero scale, never stored
                w[nt].a = w[nt].b = w[nt].c = make_uint2(0u, 0u);
                w[nt].s = 0.0f;
            }
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;

    u32x4_t xbuf[4];
    WGroup wcur[2], wnext[2];
    load_x(0, xbuf);
    load_w(0, wcur);
    store_x(0, xbuf);
    __syncthreads();

    for (int64_t g = 0; g < G; ++g) {
        const int cb = (int)(g & 1);
        const bool more = g + 1 < G;
        if (more) {
            load_x(g + 1, xbuf);
            load_w(g + 1, wnext);
        }
        // B operands: per n tile, 4 k-steps of 8 codes
        bf16x8_t bop[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const uint32_t L[4] = {wcur[nt].a.x, wcur[nt].a.y, wcur[nt].b.x, wcur[nt].b.y};
            const uint32_t H[2] = {wcur[nt].c.x, wcur[nt].c.y};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t lo16 = (L[s] >> (16 * h)) & 0xFFFFu;
                const uint32_t hi8 = (H[s >> 1] >> (16 * (s & 1) + 8 * h)) & 0xFFu;
                bop[nt][s] = eight_codes(lo16, hi8);
            }
        }
        // A operands from LDS and the MFMAs of this group
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int row = wm * 64 + mt * 32 + (lane & 31);
            bf16x8_t aop[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                aop[s] = __builtin_bit_cast(
                    bf16x8_t,
                    *reinterpret_cast<const u32x4_t*>(&xs[cb][row * XROW + 16 * s + 8 * h]));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x16_t part = {};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[s], bop[nt][s], part, 0,
                                                                  0, 0);
                const float sc = wcur[nt].s;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[mt][nt][r] = __builtin_fmaf(sc, part[r], acc[mt][nt][r]);
            }
        }
        if (more) {
            store_x(cb ^ 1, xbuf);
            wcur[0] = wnext[0];
            wcur[1] = wnext[1];
        }
        __syncthreads();
    }

    // C layout of a 32x32 tile: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            if (!orow_ok[nt]) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t t = m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (t < B) Y[t * O + orow[nt]] = acc[mt][nt][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_mfma(const uint8_t* packed, const float* scales, int64_t O,
                            int64_t I, const uint16_t* X, int64_t B, float* Y,
                            hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    const dim3 grid((unsigned)((O + BN - 1) / BN), (unsigned)((B + BM - 1) / BM));
    const bool vec = (I % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    if (vec)
        hipLaunchKernelGGL((gemm_i3_mfma_kernel<true>), grid, dim3(kThreads), 0, s, packed,
                           scales, O, I, G, X, B, Y);
    else
        hipLaunchKernelGGL((gemm_i3_mfma_kernel<false>), grid, dim3(kThreads), 0, s, packed,
                           scales, O, I, G, X, B, Y);
    return hipGetLastError();
}

}  // namespace qt
