// int3-g64 dequantize-and-multiply for batches of bf16 activations on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Y[t,o] = sum_g s[o,g] * sum_{j<64} v[o,64g+j] * X[t,64g+j]
//
// The int3 codes v in [-4,3] are exact in bf16, so each group's 64-term dot
// product is formed by the matrix cores with exact products and f32
// accumulation, then multiplied by the f32 group scale on the vector ALUs and
// added into an f32 accumulator: the per-group scale accumulation of the
// matmul_i3 kernel ("int3-g64 (fmt=5)" pull request page, "Design", Kernel
// bullet), with bf16 inputs.
//
// Tiling.  A block of 8 waves computes a BM = 256 (tokens) x BN = 144 (output
// rows) tile and walks the input dimension one 64-wide group at a time; wave w
// owns tokens [32w, 32w+32) against all 144 rows (2 x 9 MFMA tiles of 16x16).
// Per group, the block
//   * dequantizes the group's 144 x 64 codes once into LDS as bf16 (one
//     16-code quarter per thread: byte-parallel unpack, then v_perm_b32 table
//     lookups to bf16), with the 144 scales;
//   * stages the activations 256 x 64 in LDS;
// double-buffered: the loads for group g+1 are issued before the MFMAs of
// group g and written to the other buffer after them, one barrier per group.
//
// k order.  The unpack naturally yields, from a 16-code quarter, the pairs
// (0,1) (4,5) (8,9) (12,13) and (2,3) (6,7) (10,11) (14,15).  Each 8-element
// operand slice of an MFMA takes one such set, and the activations are written
// to LDS in the same order (a 32-byte load of 16 inputs is stored as its even
// and its odd 4-byte pairs), so every product pairs the right input and code
// without any shuffle.
//
// For B x O shapes that are not multiples of the tile, out-of-range rows and
// tokens read zeros (or valid addresses whose results are discarded) and are
// never stored.
#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int BM = 256;                 // tokens per block tile
constexpr int BN = 144;                 // output rows per block tile (9 x 16)
constexpr int NTN = BN / 16;            // MFMA tiles along the rows
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int ROWB = 64 * 2 + 16;       // LDS bytes per 64-element row (+16 padding)
constexpr int XS_BYTES = BM * ROWB;     // one activation buffer
constexpr int WS_BYTES = BN * ROWB;     // one dequantized-weight buffer
constexpr int kXTasks = BM * 4;         // 16-input quarters of activations per group
constexpr int kWTasks = BN * 4;         // 16-code quarters of weights per group
constexpr int kXPer = kXTasks / kThreads;                   // 2
constexpr int kWPer = (kWTasks + kThreads - 1) / kThreads;  // 2 (second for 64 threads)

// LDS byte offset, inside a 64-element row, of the 8-element slice that holds
// set `half` (0: pairs 0,1 4,5 8,9 12,13; 1: the other pairs) of quarter q.
__device__ __forceinline__ int slice_off(int q, int half) {
    const int s = q >> 1, h4 = 2 * (q & 1) + half;
    return (32 * s + 8 * h4) * 2;
}

// bf16 bit patterns of v = u - 4 for four codes u (one per byte), as the pairs
// [c0 | c1 << 16] and [c2 | c3 << 16].  bf16(v) for v = -4..3 is c080 c040 c000
// bf80 0000 3f80 4000 4040: one table gives the high bytes, one the low bytes.
__device__ __forceinline__ void to_bf16_pairs(uint32_t W4, uint32_t& d0, uint32_t& d1) {
    const uint32_t hi = __builtin_amdgcn_perm(0x40403F00u, 0xBFC0C0C0u, W4);
    const uint32_t lo = __builtin_amdgcn_perm(0x40008000u, 0x80004080u, W4);
    d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// One 16-code quarter: low-plane word L (code 4b+i at bits 8b+2i) and its 16
// high bits h16 (code j at bit j) -> set 0 and set 1 as bf16x8 (4 dwords each).
__device__ __forceinline__ void dequant_quarter(uint32_t L, uint32_t h16, u32x4_t& set0,
                                                u32x4_t& set1) {
    uint32_t sp = (h16 | (h16 << 8)) & 0x00FF00FFu;
    sp = ((sp | (sp << 4)) & 0x0F0F0F0Fu) << 2;  // code 4b+i's high bit at bit 2+i of byte b
    const uint32_t u0 = (L & 0x03030303u) | (sp & 0x04040404u);
    const uint32_t u1 = ((L >> 2) & 0x03030303u) | ((sp >> 1) & 0x04040404u);
    const uint32_t u2 = ((L >> 4) & 0x03030303u) | ((sp >> 2) & 0x04040404u);
    const uint32_t u3 = ((L >> 6) & 0x03030303u) | ((sp >> 3) & 0x04040404u);
    // natural pairs: bytes [u_i.b, u_{i+1}.b] for b = 0, 1 and b = 2, 3
    const uint32_t a0 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);  // codes 0 1 4 5
    const uint32_t a1 = __builtin_amdgcn_perm(u1, u0, 0x07030602u);  // codes 8 9 12 13
    const uint32_t b0 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);  // codes 2 3 6 7
    const uint32_t b1 = __builtin_amdgcn_perm(u3, u2, 0x07030602u);  // codes 10 11 14 15
    uint32_t d[8];
    to_bf16_pairs(a0, d[0], d[1]);
    to_bf16_pairs(a1, d[2], d[3]);
    to_bf16_pairs(b0, d[4], d[5]);
    to_bf16_pairs(b1, d[6], d[7]);
    set0 = u32x4_t{d[0], d[1], d[2], d[3]};
    set1 = u32x4_t{d[4], d[5], d[6], d[7]};
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_i3_mfma_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int64_t I,
    int64_t G, const uint16_t* __restrict__ X, int64_t B, float* __restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* xs = smem;                           // [2][BM][ROWB]
    uint8_t* ws = smem + 2 * XS_BYTES;            // [2][BN][ROWB]
    float* ss = reinterpret_cast<float*>(smem + 2 * XS_BYTES + 2 * WS_BYTES);  // [2][BN]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h4 = lane >> 4;  // which 8-element slice of an MFMA operand
    const int l16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;

    // ---- loaders (branch-free: out-of-range pieces load a valid address and
    // are replaced by zeros or discarded).  Per-thread base pointers are set
    // up once; each group only advances them.
    const uint16_t* xrow[kXPer];
    bool xrow_ok[kXPer];
    int xq16[kXPer];
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
        const int task = tid + kThreads * i;
        const int64_t t = m0 + (task >> 2);
        xrow_ok[i] = t < B;
        xq16[i] = 16 * (task & 3);
        xrow[i] = X + (xrow_ok[i] ? t : 0) * I + xq16[i];
    }
    const uint8_t* wrow[kWPer];
    const float* srow[kWPer];
    bool w_ok[kWPer];
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
        const int task = tid + kThreads * i;
        const int64_t n = n0 + (task >> 2);
        w_ok[i] = task < kWTasks && n < O;
        const int64_t gi = w_ok[i] ? n * G : 0;
        wrow[i] = packed + gi * kGroupBytes + 4 * (task & 3);
        srow[i] = scales + gi;
    }

    // Raw loaded values stay untouched until the store after the MFMAs:
    // anything computed from them right after the load would make the wave
    // wait for the data there.
    struct XLoad {
        u32x4_t a, b;
        bool ok0, ok1;
    };
    auto load_x = [&](int64_t g, XLoad (&xl)[kXPer]) {
#pragma unroll
        for (int i = 0; i < kXPer; ++i) {
            const int64_t k = g * kGroup + xq16[i];  // first input of the quarter
            const uint16_t* src = xrow[i] + g * kGroup;
            if constexpr (VEC) {
                xl[i].ok0 = xrow_ok[i] && k < I;
                xl[i].ok1 = xrow_ok[i] && k + 8 < I;
                xl[i].a = *reinterpret_cast<const u32x4_t*>(xl[i].ok0 ? src : X);
                xl[i].b = *reinterpret_cast<const u32x4_t*>(xl[i].ok1 ? src + 8 : X);
            } else {
                // unaligned rows: element loads, masked here (rare path)
                uint32_t w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool oa = xrow_ok[i] && k + 2 * e < I;
                    const bool ob = xrow_ok[i] && k + 2 * e + 1 < I;
                    const uint32_t va = *(oa ? src + 2 * e : X);
                    const uint32_t vb = *(ob ? src + 2 * e + 1 : X);
                    w[e] = (oa ? va : 0u) | ((ob ? vb : 0u) << 16);
                }
                xl[i].a = u32x4_t{w[0], w[1], w[2], w[3]};
                xl[i].b = u32x4_t{w[4], w[5], w[6], w[7]};
                xl[i].ok0 = xl[i].ok1 = true;
            }
        }
    };
    // store: the 16 inputs of a quarter as their even pairs (set 0) and odd
    // pairs (set 1); pieces past the row or the batch become zeros
    auto store_x = [&](int buf, const XLoad (&xl)[kXPer]) {
#pragma unroll
        for (int i = 0; i < kXPer; ++i) {
            const int task = tid + kThreads * i;
            const int row = task >> 2, q = task & 3;
            uint8_t* r = xs + buf * XS_BYTES + row * ROWB;
            const u32x4_t z = {0u, 0u, 0u, 0u};
            const u32x4_t a = xl[i].ok0 ? xl[i].a : z;
            const u32x4_t b = xl[i].ok1 ? xl[i].b : z;
            const u32x4_t s0 = {a.x, a.z, b.x, b.z};
            const u32x4_t s1 = {a.y, a.w, b.y, b.w};
            *reinterpret_cast<u32x4_t*>(r + slice_off(q, 0)) = s0;
            *reinterpret_cast<u32x4_t*>(r + slice_off(q, 1)) = s1;
        }
    };
    struct WLoad {
        uint32_t lo, hw;
        float s;
    };
    auto load_w = [&](int64_t g, WLoad (&wl)[kWPer]) {
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            const int q = (tid + kThreads * i) & 3;
            // rows past O read their block's group 0 (valid); their scale is
            // replaced by 0 at the store
            const uint8_t* p = wrow[i] + (w_ok[i] ? g * kGroupBytes : 0);
            wl[i].lo = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
            wl[i].hw = __builtin_nontemporal_load(
                reinterpret_cast<const uint32_t*>(p - 4 * q + 16 + 4 * (q >> 1)));
            wl[i].s = srow[i][w_ok[i] ? g : 0];
        }
    };
    auto store_w = [&](int buf, const WLoad (&wl)[kWPer]) {
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            const int task = tid + kThreads * i;
            if (task < kWTasks) {
                const int n = task >> 2, q = task & 3;
                u32x4_t s0, s1;
                dequant_quarter(wl[i].lo, (wl[i].hw >> (16 * (q & 1))) & 0xFFFFu, s0, s1);
                uint8_t* r = ws + buf * WS_BYTES + n * ROWB;
                *reinterpret_cast<u32x4_t*>(r + slice_off(q, 0)) = s0;
                *reinterpret_cast<u32x4_t*>(r + slice_off(q, 1)) = s1;
                if (q == 0) ss[buf * BN + n] = w_ok[i] ? wl[i].s : 0.0f;
            }
        }
    };

    f32x4_t acc[2][NTN];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // MFMAs and scale accumulation of one group from LDS buffer cb.  The B
    // operands and scale of row tile nt+1 are read from LDS while tile nt is
    // multiplied, so LDS latency overlaps the matrix cores.
    auto compute = [&](int cb) {
        const uint8_t* xb = xs + cb * XS_BYTES + (wave * 32 + l16) * ROWB + 16 * h4;
        const uint8_t* wb = ws + cb * WS_BYTES + l16 * ROWB + 16 * h4;
        const float* sb = ss + cb * BN + l16;
        bf16x8_t aop[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                aop[mt][s] = __builtin_bit_cast(
                    bf16x8_t,
                    *reinterpret_cast<const u32x4_t*>(xb + mt * 16 * ROWB + 64 * s));
        bf16x8_t bcur0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(wb));
        bf16x8_t bcur1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(wb + 64));
        float scur = sb[0];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) {
            bf16x8_t bnext0 = bcur0, bnext1 = bcur1;
            float snext = scur;
            if (nt + 1 < NTN) {
                const uint8_t* wr = wb + (nt + 1) * 16 * ROWB;
                bnext0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(wr));
                bnext1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(wr + 64));
                snext = sb[(nt + 1) * 16];
            }
            f32x4_t part[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                part[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    aop[mt][0], bcur0, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                part[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[mt][1], bcur1, part[mt], 0,
                                                                   0, 0);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[mt][nt][r] = __builtin_fmaf(scur, part[mt][r], acc[mt][nt][r]);
            bcur0 = bnext0;
            bcur1 = bnext1;
            scur = snext;
        }
    };

    // Software pipeline.  The packed weights stream from HBM and are fetched
    // two groups ahead (group g+1 waits in registers while g+2 is in flight);
    // the activations, which every block re-reads and mostly hit L2, are
    // fetched one group ahead.  After the MFMAs of group g, group g+1 is
    // dequantized and stored into the other LDS buffer.
    // The loop body is straight-line (prefetches past the last group re-read
    // group G-1 and land in a buffer nobody reads): with loads issued under
    // conditions the compiler cannot tell which are still in flight and waits
    // for all of them.
    XLoad xl[kXPer];
    WLoad wa[kWPer], wb[kWPer];
    const int64_t glast = G - 1;
    load_x(0, xl);
    load_w(0, wa);
    store_x(0, xl);
    store_w(0, wa);
    load_w(min<int64_t>(1, glast), wa);
    __syncthreads();
    for (int64_t g = 0;; g += 2) {
        // step g: registers A hold group g+1's weights, fetch g+2's
        load_x(min(g + 1, glast), xl);
        load_w(min(g + 2, glast), wb);
        compute(0);
        store_x(1, xl);
        store_w(1, wa);
        __syncthreads();
        if (g + 1 >= G) break;
        // step g+1: registers B hold group g+2's weights, fetch g+3's
        load_x(min(g + 2, glast), xl);
        load_w(min(g + 3, glast), wa);
        compute(1);
        store_x(0, xl);
        store_w(0, wb);
        __syncthreads();
        if (g + 2 >= G) break;
    }

    // C layout of a 16x16 tile: register r of lane l holds token row
    // 4*(l/16) + r and output column l%16.
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt) {
        const int64_t o = n0 + nt * 16 + l16;
        if (o >= O) continue;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = m0 + wave * 32 + mt * 16 + 4 * h4 + r;
                if (t < B) Y[t * O + o] = acc[mt][nt][r];
            }
    }
}

constexpr size_t kSmem = 2 * XS_BYTES + 2 * WS_BYTES + 2 * BN * sizeof(float);

}  // namespace

hipError_t launch_gemm_mfma(const uint8_t* packed, const float* scales, int64_t O,
                            int64_t I, const uint16_t* X, int64_t B, float* Y,
                            hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    const dim3 grid((unsigned)((O + BN - 1) / BN), (unsigned)((B + BM - 1) / BM));
    const bool vec = (I % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    hipError_t e;
    if (vec) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_i3_mfma_kernel<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((gemm_i3_mfma_kernel<true>), grid, dim3(kThreads), kSmem, s, packed,
                           scales, O, I, G, X, B, Y);
    } else {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_i3_mfma_kernel<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((gemm_i3_mfma_kernel<false>), grid, dim3(kThreads), kSmem, s, packed,
                           scales, O, I, G, X, B, Y);
    }
    return hipGetLastError();
}

}  // namespace qt
