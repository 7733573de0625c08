// The grouped (mixture-of-experts) matrix-core tile shared by the grouped
// multiply and the MoE expert layer; see grouped.hip for the method.
#pragma once
#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kRows = 64;             // output rows per block
constexpr int kThreads = 256;         // 4 waves
constexpr int kTok = 5;               // tokens per pass (3 B columns each)

// Chunk geometry: CG groups per chunk (8 or 16), LDS bytes per piece column,
// scales staged per thread.
template <int CG>
struct Chunking {
    static constexpr int kCG = CG;
    static constexpr int kPRow = CG * kGroup * 2 + 16;
    static constexpr int kSPer = kRows * CG / kThreads;
    static_assert(CG == 8 || CG == 16, "8 or 16 groups per chunk");
};

// Weight staging geometry of a format: bytes per group, LDS bytes per weight
// row (+16: conflict-free reads), 16-byte pieces per thread per chunk.
template <int BITS, int CG>
struct Geo {
    static constexpr int kGB = BITS == 3 ? kGroupBytes : kGroupBytesI4;
    static constexpr int kWRow = CG * kGB + 16;
    static constexpr int kWPieces = kRows * CG * kGB / 16;  // 768..2048
    static constexpr int kWPer = kWPieces / kThreads;       // 3..8
    static_assert(kWPieces % kThreads == 0, "weight chunk split");
};

// One 16-code quarter: low-plane word L (code 4b+i at bits 8b+2i) and the
// 32-bit high-plane word hw holding its 16 high bits (bytes 0-1 or 2-3, as
// hsel selects: code j at bit j) -> its codes v as bf16, in the k order the
// int3 tile stages its inputs in: lo8 holds codes 0 4 1 5 2 6 3 7 and hi8
// codes 8 12 9 13 10 14 11 15 of the quarter (a dot product does not depend
// on the order of its terms, only on both operands using the same one).
//   * one byte permute puts the quarter's two high bytes in bytes 0 and 2,
//     and one shift-or spreads nibble b to byte b: bit i of byte b is then
//     the high bit of code 4b+i;
//   * u_i = ((L >> 2i) & 3) | (high bit << 2) per byte is u = v + 4 of code
//     4b+i in byte b;
//   * a byte-permute table maps each u to the FP8 (E4M3) encoding of v/256:
//     sign and magnitude, |v| <= 3 as the subnormal 2|v| * 2^-9 and -4 as the
//     smallest normal 2^-6 (bytes 88 86 84 82 00 02 04 06 for u = 0..7);
//   * the conversion of two FP8 bytes to bf16 with the scale 2^8 gives
//     bf16(v) exactly, two codes per instruction.
__device__ __forceinline__ void dequant_quarter(uint32_t L, uint32_t hw, uint32_t hsel,
                                                u32x4_t& lo8, u32x4_t& hi8) {
    const uint32_t b = __builtin_amdgcn_perm(0u, hw, hsel);
    const uint32_t t = (b | (b << 4)) & 0x0F0F0F0Fu;  // bit i of byte b: high bit of 4b+i
    uint32_t f[4];
    f[0] = (L & 0x03030303u) | ((t << 2) & 0x04040404u);
    f[1] = ((L >> 2) & 0x03030303u) | ((t << 1) & 0x04040404u);
    f[2] = ((L >> 4) & 0x03030303u) | (t & 0x04040404u);
    f[3] = ((L >> 6) & 0x03030303u) | ((t >> 1) & 0x04040404u);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __builtin_amdgcn_perm(0x06040200u, 0x82848688u, f[i]);
    // byte b of f_i is code 4b+i: pairs (i, 4+i) from bytes 0-1, (8+i, 12+i)
    // from bytes 2-3
#define QT_CV(u, HI) \
    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u, 256.0f, HI))
    lo8 = u32x4_t{QT_CV(f[0], false), QT_CV(f[1], false), QT_CV(f[2], false), QT_CV(f[3], false)};
    hi8 = u32x4_t{QT_CV(f[0], true), QT_CV(f[1], true), QT_CV(f[2], true), QT_CV(f[3], true)};
#undef QT_CV
}

// v/16 of the two's-complement nibble in the low four bits of byte B of t.
template <int B>
__device__ __forceinline__ float nib(uint32_t t) {
    float r;
    if constexpr (B == 0)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
            : "=v"(r) : "v"(t));
    else if constexpr (B == 1)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
            : "=v"(r) : "v"(t));
    else if constexpr (B == 2)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2"
            : "=v"(r) : "v"(t));
    else
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
            : "=v"(r) : "v"(t));
    return r;
}

// bf16 pair [f(a) | f(b) << 16] of two f32 values with zero low halves.
__device__ __forceinline__ uint32_t hi_pair(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// One int4 word (code n of the word in nibble n, u = v + 8) -> its 8 codes
// as v/16 in bf16, natural order.  u ^ 8 is the two's-complement nibble of v.
__device__ __forceinline__ u32x4_t dequant_word_i4(uint32_t w) {
    const uint32_t t = w ^ 0x88888888u;  // even codes: low nibble of each byte
    const uint32_t h = t >> 4;           // odd codes: low nibble of each byte
    return u32x4_t{hi_pair(nib<0>(t), nib<0>(h)), hi_pair(nib<1>(t), nib<1>(h)),
                   hi_pair(nib<2>(t), nib<2>(h)), hi_pair(nib<3>(t), nib<3>(h))};
}

// The three bf16 pieces of four f32 inputs, as [piece][pair] words.
__device__ __forceinline__ void split3(const float (&x)[4], uint32_t (&w)[3][2]) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float hf = __uint_as_float(__float_as_uint(x[e]) & 0xFFFF0000u);
        const float r1 = x[e] - hf;
        const float mf = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
        const float lf = r1 - mf;
        h[e] = __float_as_uint(hf);
        m[e] = __float_as_uint(mf);
        l[e] = __float_as_uint(lf);
    }
    // high halves of two words -> one word (element 2k in the low half)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        w[0][k] = __builtin_amdgcn_perm(h[2 * k + 1], h[2 * k], 0x07060302u);
        w[1][k] = __builtin_amdgcn_perm(m[2 * k + 1], m[2 * k], 0x07060302u);
        w[2][k] = __builtin_amdgcn_perm(l[2 * k + 1], l[2 * k], 0x07060302u);
    }
}

// lane l takes the value of lane l + M of its 16-lane row (0 past the row)
template <int M>
__device__ __forceinline__ float from_lane_plus(float a) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0x100 + M, 0xF, 0xF, true));
}

// LDS of one tile; WROW: weight bytes per row (the larger format's for a
// kernel that runs both), CG groups per chunk.
template <int WROW, int CG>
struct TileLds {
    __attribute__((aligned(16))) uint8_t wl[kRows * WROW];   // weight bytes
    __attribute__((aligned(16))) float sl[CG][kRows];        // scales [group][row]
    __attribute__((aligned(16))) uint8_t pl[16 * Chunking<CG>::kPRow];  // pieces [col][k]
    int32_t trow[kTok];
    int32_t tout[kTok];
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// One item: the pairs of expert e against its rows [64 rb, 64 rb + 64).
// W16: every row's chunk bytes start on a 16-byte boundary (int4, or int3
// with G even); else 8-byte pieces.  XV: inputs allow 16-byte loads
// (I % 4 == 0, X 16-byte aligned).  Starts with a barrier, so items can
// follow one another in a block.
template <int BITS, bool W16, bool XV, int WROW, int CG>
__device__ __forceinline__ void grouped_tile(
    TileLds<WROW, CG>& L, int e, int64_t rb, const uint8_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t O, int32_t I, int32_t G,
    const float* __restrict__ X, int64_t n_x_rows,
    const int32_t* __restrict__ pair_row, const int32_t* __restrict__ off, int32_t P,
    float* __restrict__ Y) {
    constexpr int kGB = Geo<BITS, CG>::kGB;
    constexpr int kWRow = Geo<BITS, CG>::kWRow;
    constexpr int kWPer = Geo<BITS, CG>::kWPer;
    constexpr int kCG = CG;
    constexpr int kPRow = Chunking<CG>::kPRow;
    constexpr int kSPer = Chunking<CG>::kSPer;
    // Weights are read once: non-temporal loads keep them out of the caches,
    // but only where a row's chunk is whole 128-byte lines; otherwise the line
    // that two consecutive chunks share would be fetched twice.
    constexpr bool kStream = (kCG * kGB) % 128 == 0;
    static_assert(kWRow <= WROW, "tile LDS too small for the format");
    uint8_t* wl = L.wl;
    auto& sl = L.sl;
    uint8_t* pl = L.pl;
    int32_t* trow = L.trow;
    int32_t* tout = L.tout;

    const int32_t p0 = max(0, min(off[e], P));
    const int32_t p1 = max(p0, min(off[e + 1], P));
    if (p1 == p0) return;  // uniform over the block
    __syncthreads();  // an earlier item of this block is done with the LDS

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int j4 = lane >> 4;  // quarter of the group (A), k slot (B)
    const int64_t r0 = rb * kRows;
    const uint8_t* pk = packed + (int64_t)e * O * G * kGB;
    const float* sk = scales + (int64_t)e * O * G;

    // column 15 of the pieces is never written by the staging: zero it once
    for (int i = tid; i < kCG * kGroup / 2; i += kThreads)
        reinterpret_cast<uint32_t*>(pl + 15 * kPRow)[i] = 0u;

    // ---- per-thread staging assignments (rows past O read row O-1, unused)
    // weights: piece i of this thread = 16-byte piece (tid + 256 i) of the
    // chunk, row-major over [row][kCG * kGB bytes]
    const uint8_t* wrow0[kWPer];  // the row's first byte (always a valid 16 bytes)
    int wdst[kWPer];
    int wpart[kWPer];
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
        const int id = tid + kThreads * i;
        const int row = id / (kCG * kGB / 16), part = id % (kCG * kGB / 16);
        const int64_t gr = min<int64_t>(r0 + row, O - 1);
        wrow0[i] = pk + gr * G * kGB;
        wdst[i] = row * kWRow + 16 * part;
        wpart[i] = part;
    }
    // scales: kSPer per thread, [row][CG groups] -> sl[group][row]
    const int srow = tid / (kCG / kSPer), sg = (tid % (kCG / kSPer)) * kSPer;
    const bool xq = 4 * tid < kCG * kGroup;  // this thread stages 4 inputs
    const float* ssrc = sk + min<int64_t>(r0 + srow, O - 1) * G;

    struct Chunk {
        u32x4_t w[kWPer];
        float s[kSPer];
        float x[kTok][4];
    };
    auto load_chunk = [&](int32_t c0, int nt, Chunk& c) {
        const int gn = min(kCG, G - c0);
        // pieces past the chunk's bytes re-read the row's first 16 bytes
        // (unused); with G even every piece lies wholly inside or outside
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            const int b0 = wpart[i] * 16;
            const uint8_t* rc = wrow0[i] + (int64_t)c0 * kGB;
            if constexpr (W16) {
                const uint8_t* src = b0 < gn * kGB ? rc + b0 : wrow0[i];
                const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(src);
                c.w[i] = kStream ? __builtin_nontemporal_load(sp) : *sp;
            } else {
                static_assert(BITS == 3, "int4 groups are always 16-byte aligned");
                const uint8_t* sa = b0 < gn * kGB ? rc + b0 : wrow0[i];
                const uint8_t* sb = b0 + 8 < gn * kGB ? rc + b0 + 8 : wrow0[i];
                const u32x2_t* pa = reinterpret_cast<const u32x2_t*>(sa);
                const u32x2_t* pb = reinterpret_cast<const u32x2_t*>(sb);
                const u32x2_t a = kStream ? __builtin_nontemporal_load(pa) : *pa;
                const u32x2_t b = kStream ? __builtin_nontemporal_load(pb) : *pb;
                c.w[i] = u32x4_t{a.x, a.y, b.x, b.y};
            }
        }
#pragma unroll
        for (int q = 0; q < kSPer; ++q) c.s[q] = ssrc[min(c0 + sg + q, G - 1)];
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            if (t >= nt) break;  // uniform
            const int64_t xr = trow[t];
            const int32_t k0 = c0 * kGroup + 4 * tid;  // this thread's 4 inputs
            const float* src = X + xr * I;
            if constexpr (XV) {
                const bool ok = k0 < I;
                const float4 v = *reinterpret_cast<const float4*>(src + (ok ? k0 : 0));
                c.x[t][0] = v.x;
                c.x[t][1] = v.y;
                c.x[t][2] = v.z;
                c.x[t][3] = v.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) c.x[t][q] = src[k0 + q < I ? k0 + q : 0];
            }
        }
    };
    auto store_chunk = [&](int32_t c0, int nt, const Chunk& c) {
        const int gn = min(kCG, G - c0);
#pragma unroll
        for (int i = 0; i < kWPer; ++i)
            *reinterpret_cast<u32x4_t*>(wl + wdst[i]) = c.w[i];
#pragma unroll
        for (int q = 0; q < kSPer; ++q) sl[sg + q][srow] = sg + q < gn ? c.s[q] : 0.0f;
        const int32_t k0 = c0 * kGroup + 4 * tid;
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            if (t < nt && xq) {  // t < nt uniform; columns of absent tokens stay zero
                float x[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = k0 + q < I ? c.x[t][q] : 0.0f;
                if constexpr (BITS == 3) {
                    // aligned 8-input block = this thread's 4 and its
                    // neighbour's; position 2i holds input i, 2i+1 input 4+i
                    float pn[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        pn[q] = __int_as_float(__builtin_amdgcn_update_dpp(
                            0, __float_as_int(x[q]), 0xB1, 0xF, 0xF, false));  // lane ^ 1
                    const bool odd = tid & 1;
                    const float y0 = odd ? pn[2] : x[0], y1 = odd ? x[2] : pn[0];
                    const float y2 = odd ? pn[3] : x[1], y3 = odd ? x[3] : pn[1];
                    x[0] = y0;
                    x[1] = y1;
                    x[2] = y2;
                    x[3] = y3;
                }
                uint32_t w[3][2];
                split3(x, w);
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    *reinterpret_cast<u32x2_t*>(pl + (3 * t + p) * kPRow + 8 * tid) =
                        u32x2_t{w[p][0], w[p][1]};
            }
        }
    };

    for (int32_t pb = p0; pb < p1; pb += kTok) {
        const int nt = min(kTok, p1 - pb);
        __syncthreads();  // the previous pass is done with trow/tout and LDS
        if (tid < kTok) {
            const int32_t p = pb + min(tid, nt - 1);
            const int32_t xr = pair_row ? pair_row[p] : p;
            // out-of-range rows read row 0 and are not written; the host
            // documents the valid range, this only keeps accesses in bounds
            const bool ok = xr >= 0 && xr < n_x_rows && tid < nt;
            trow[tid] = (xr >= 0 && xr < n_x_rows) ? xr : 0;
            tout[tid] = ok ? pb + tid : -1;
        }
        __syncthreads();

        // columns of tokens past nt read zeros for the whole pass
        for (int i = tid; i < (3 * (kTok - nt)) * (kCG * kGroup / 2); i += kThreads) {
            const int col = 3 * nt + i / (kCG * kGroup / 2), w = i % (kCG * kGroup / 2);
            reinterpret_cast<uint32_t*>(pl + col * kPRow)[w] = 0u;
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        Chunk cur;
        load_chunk(0, nt, cur);
        for (int32_t c0 = 0; c0 < G; c0 += kCG) {
            const int gn = min(kCG, G - c0);
            __syncthreads();  // everyone is done with the previous chunk
            store_chunk(c0, nt, cur);
            __syncthreads();
            // next chunk in flight while this one is multiplied
            if (c0 + kCG < G) load_chunk(c0 + kCG, nt, cur);
            const uint8_t* wrow = wl + (16 * wave + l16) * kWRow;
            const uint8_t* prow = pl + l16 * kPRow + 32 * j4;
            // selector of the quarter's two high-plane bytes (int3)
            const uint32_t hsel = (j4 & 1) ? 0x0c030c02u : 0x0c010c00u;
#pragma unroll
            for (int g = 0; g < kCG; ++g) {
                if (g >= gn) break;  // uniform
                u32x4_t a0, a1;
                if constexpr (BITS == 3) {
                    const uint32_t lo =
                        *reinterpret_cast<const uint32_t*>(wrow + g * kGB + 4 * j4);
                    const uint32_t hw = *reinterpret_cast<const uint32_t*>(
                        wrow + g * kGB + 16 + 4 * (j4 >> 1));
                    dequant_quarter(lo, hw, hsel, a0, a1);
                } else {
                    // quarter j4 = codes 16 j4 .. 16 j4 + 15 = bytes 8 j4 .. 8 j4 + 7
                    const u32x2_t q = *reinterpret_cast<const u32x2_t*>(wrow + g * kGB + 8 * j4);
                    a0 = dequant_word_i4(q.x);
                    a1 = dequant_word_i4(q.y);
                }
                const u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(prow + g * 128);
                const u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(prow + g * 128 + 16);
                f32x4_t part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, b0),
                    f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, b1), part, 0,
                    0, 0);
                const f32x4_t s4 =
                    *reinterpret_cast<const f32x4_t*>(&sl[g][16 * wave + 4 * j4]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(s4[r], part[r], acc[r]);
            }
        }
        // C layout: register r of lane l holds row 4*(l/16)+r of the wave's
        // tile and column l%16 = 3t + piece; lane 3t adds its two neighbours
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v1 = from_lane_plus<1>(acc[r]);
            const float v2 = from_lane_plus<2>(acc[r]);
            acc[r] = (acc[r] + v1) + v2;
            if constexpr (BITS == 4) acc[r] *= 16.0f;  // the codes entered as v/16
        }
        const int t = l16 / 3;
        if (l16 % 3 == 0 && t < nt && tout[t] >= 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t o = r0 + 16 * wave + 4 * j4 + r;
                if (o < O) Y[(int64_t)tout[t] * O + o] = acc[r];
            }
        }
    }
}

}  // namespace
}  // namespace qt
