// The grouped (mixture-of-experts) matrix-core tile shared by the grouped
// multiply and the MoE expert layer; see grouped.hip for the method.
#pragma once
#include <type_traits>

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

// The three bf16 pieces of E f32 inputs, as [piece][pair] words.
template <int E>
__device__ __forceinline__ void split3(const float (&x)[E], uint32_t (&w)[3][E / 2]) {
    uint32_t h[E], m[E], l[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
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
    for (int k = 0; k < E / 2; ++k) {
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

// Inputs per thread per chunk: all 256 threads stage the chunk's CG * 64.
template <int CG>
constexpr int kXPer = CG * kGroup / kThreads;

// A chunk's scales and this thread's inputs, in registers between their
// loads and their stores to LDS.
template <int CG>
struct SxRegs {
    float s[Chunking<CG>::kSPer];
    float x[kTok][kXPer<CG>];
};

// Per-thread roles in staging scales and inputs: scales of row srow, groups
// sg .. sg + kSPer - 1 of each chunk (rows past O read row O - 1, unused);
// the inputs of positions E tid .. E tid + E - 1 of each chunk's staged
// order (E = kXPer).
template <int CG>
struct SxRoles {
    int srow, sg;
    const float* ssrc;
    __device__ __forceinline__ SxRoles(int tid, const float* sk, int64_t r0, int64_t O,
                                       int32_t G) {
        constexpr int kSPer = Chunking<CG>::kSPer;
        srow = tid / (CG / kSPer);
        sg = (tid % (CG / kSPer)) * kSPer;
        ssrc = sk + min<int64_t>(r0 + srow, O - 1) * G;
    }
};

// The input (offset in the chunk) at position P of the staged order: the
// natural order for int4; for int3 the order the table unpacking yields the
// codes in, 0 4 1 5 2 6 3 7 within each aligned eight.
template <int BITS>
__device__ __forceinline__ int staged_input(int P) {
    if constexpr (BITS == 4) {
        return P;
    } else {
        const int r = P & 7;
        return (P & ~7) + ((r & 1) ? 4 + (r >> 1) : (r >> 1));
    }
}

// Rows of the pass's tokens in X, as block-uniform pointers (the row
// arithmetic runs once per pass, on the scalar unit).
__device__ __forceinline__ void token_rows(const int32_t* trow, const float* __restrict__ X,
                                           int32_t I, int nt, const float* (&xrow)[kTok]) {
#pragma unroll
    for (int t = 0; t < kTok; ++t)
        xrow[t] = X + (int64_t)__builtin_amdgcn_readfirstlane(trow[t < nt ? t : 0]) * I;
}

// FULL: the chunk's CG groups and CG * 64 inputs all lie inside the matrix
// (every chunk but a short last one), so no index needs clamping.  XV loads
// runs of consecutive inputs as vectors (int4: E at once; int3: E = 4 as
// inputs 2j, 2j + 1 and 4 + 2j, 5 + 2j of an eight), each wholly inside or
// outside the row since I % 4 == 0; one past the row reads the row's first
// inputs instead (zeroed when stored).
template <int BITS, int CG, bool XV, bool FULL>
__device__ __forceinline__ void load_sx(SxRegs<CG>& c, const SxRoles<CG>& ro, int32_t c0,
                                        const float* const (&xrow)[kTok], int32_t I, int32_t G,
                                        int tid) {
    constexpr int E = kXPer<CG>;
    static_assert(E == 2 || E == 4, "two or four inputs per thread");
#pragma unroll
    for (int q = 0; q < Chunking<CG>::kSPer; ++q)
        c.s[q] = ro.ssrc[FULL ? c0 + ro.sg + q : min(c0 + ro.sg + q, G - 1)];
    const int32_t k0 = c0 * kGroup;
    // offset of input k of the chunk from the chunk's start (clamped: past
    // the row, the row's first input)
    auto at = [&](int k) { return FULL || (int64_t)k0 + k < I ? k : -k0; };
    // Every token slot loads (slots past nt read token 0's row, unused): with
    // an early exit at nt the compiler copied the loaded registers between
    // the exit paths, and such a copy waits for every load in flight, the
    // next chunk's weights included, before the multiply could start.
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        const float* src = xrow[t] + k0;  // uniform
        if constexpr (XV && BITS == 4 && E == 4) {
            const float4 v = *reinterpret_cast<const float4*>(src + at(4 * tid));
            c.x[t][0] = v.x;
            c.x[t][1] = v.y;
            c.x[t][2] = v.z;
            c.x[t][3] = v.w;
        } else if constexpr (XV && BITS == 4) {
            const float2 v = *reinterpret_cast<const float2*>(src + at(2 * tid));
            c.x[t][0] = v.x;
            c.x[t][1] = v.y;
        } else if constexpr (XV && E == 4) {
            const int b = 8 * (tid >> 1) + 2 * (tid & 1);
            const float2 lo = *reinterpret_cast<const float2*>(src + at(b));
            const float2 hi = *reinterpret_cast<const float2*>(src + at(b + 4));
            c.x[t][0] = lo.x;
            c.x[t][1] = hi.x;
            c.x[t][2] = lo.y;
            c.x[t][3] = hi.y;
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) c.x[t][e] = src[at(staged_input<BITS>(E * tid + e))];
        }
    }
}

// Scales to sl[group][row] (zero past the last group) and the bf16 pieces
// of the live tokens' inputs to pl (column 3t + piece, positions E tid ..
// E tid + E - 1; inputs past I as zeros).
template <int BITS, int CG, bool FULL>
__device__ __forceinline__ void store_sx(const SxRegs<CG>& c, const SxRoles<CG>& ro, int32_t c0,
                                         int nt, float (*sl)[kRows], uint8_t* pl, int32_t I,
                                         int32_t G, int tid) {
    constexpr int kPRow = Chunking<CG>::kPRow;
    constexpr int E = kXPer<CG>;
    const int gn = min(CG, G - c0);
#pragma unroll
    for (int q = 0; q < Chunking<CG>::kSPer; ++q)
        sl[ro.sg + q][ro.srow] = FULL || ro.sg + q < gn ? c.s[q] : 0.0f;
    const int32_t k0 = c0 * kGroup;
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        if (t >= nt) break;  // uniform; columns of absent tokens stay zero
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            x[e] = FULL || (int64_t)k0 + staged_input<BITS>(E * tid + e) < I ? c.x[t][e] : 0.0f;
        uint32_t w[3][E / 2];
        split3<E>(x, w);
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            uint8_t* dst = pl + (3 * t + p) * kPRow + 2 * E * tid;
            if constexpr (E == 4)
                *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w[p][0], w[p][1]};
            else
                *reinterpret_cast<uint32_t*>(dst) = w[p][0];
        }
    }
}

// The gn groups of one chunk staged in LDS (weights wl at the format's row
// pitch, pieces pl, scales sl) into acc: per group two MFMAs over the exact
// codes and the pieces, then one FMA with the row's scale.
template <int BITS, int CG>
__device__ __forceinline__ void mma_chunk(const uint8_t* wl, const uint8_t* pl,
                                          const float (*sl)[kRows], int gn, int wave, int l16,
                                          int j4, f32x4_t& acc) {
    constexpr int kGB = Geo<BITS, CG>::kGB;
    constexpr int kWRow = Geo<BITS, CG>::kWRow;
    constexpr int kPRow = Chunking<CG>::kPRow;
    const uint8_t* wrow = wl + (16 * wave + l16) * kWRow;
    const uint8_t* prow = pl + l16 * kPRow + 32 * j4;
    // selector of the quarter's two high-plane bytes (int3)
    const uint32_t hsel = (j4 & 1) ? 0x0c030c02u : 0x0c010c00u;
#pragma unroll
    for (int g = 0; g < CG; ++g) {
        if (g >= gn) break;  // uniform
        u32x4_t a0, a1;
        if constexpr (BITS == 3) {
            const uint32_t lo = *reinterpret_cast<const uint32_t*>(wrow + g * kGB + 4 * j4);
            const uint32_t hw =
                *reinterpret_cast<const uint32_t*>(wrow + g * kGB + 16 + 4 * (j4 >> 1));
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
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                       __builtin_bit_cast(bf16x8_t, b1), part, 0,
                                                       0, 0);
        const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(&sl[g][16 * wave + 4 * j4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(s4[r], part[r], acc[r]);
    }
}

// C layout: register r of lane l holds row 4*(l/16)+r of the wave's tile and
// column l%16 = 3t + piece; lane 3t adds its two neighbours and writes the
// rows of token t.
template <int BITS>
__device__ __forceinline__ void store_rows(f32x4_t acc, int nt, const int32_t* tout, int64_t r0,
                                           int64_t O, int wave, int l16, int j4,
                                           float* __restrict__ Y) {
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

// Rows of the pass's tokens (pairs pb .. pb + nt - 1) into trow/tout; the
// caller has passed a barrier since the previous pass last read them.
__device__ __forceinline__ void pass_tokens(int32_t* trow, int32_t* tout, int32_t pb, int nt,
                                            const int32_t* __restrict__ pair_row,
                                            int64_t n_x_rows, int tid) {
    if (tid < kTok) {
        const int32_t p = pb + min(tid, nt - 1);
        const int32_t xr = pair_row ? pair_row[p] : p;
        // out-of-range rows read row 0 and are not written; the host
        // documents the valid range, this only keeps accesses in bounds
        const bool ok = xr >= 0 && xr < n_x_rows && tid < nt;
        trow[tid] = (xr >= 0 && xr < n_x_rows) ? xr : 0;
        tout[tid] = ok ? pb + tid : -1;
    }
}

// Zero the piece columns of tokens nt .. kTok - 1 for the whole pass, and
// column 15, which no token uses.
template <int CG>
__device__ __forceinline__ void zero_columns(uint8_t* pl, int nt, int tid) {
    constexpr int kPRow = Chunking<CG>::kPRow;
    constexpr int kW = CG * kGroup / 2;  // 32-bit words of one column
    for (int i = tid; i < (3 * (kTok - nt) + 1) * kW; i += kThreads) {
        const int col = 3 * nt + i / kW, w = i % kW;
        reinterpret_cast<uint32_t*>(pl + col * kPRow)[w] = 0u;  // col <= 3 kTok = 15
    }
}

// One item: the pairs of expert e against its rows [64 rb, 64 rb + 64).
// W16: every row's chunk bytes start on a 16-byte boundary (int4, or int3
// with G even); else 8-byte pieces.  XV: inputs allow 16-byte loads
// (I % 4 == 0, X 16-byte aligned).  Full chunks take loads and stores
// without clamping, in code of their own.  Starts with a barrier, so items
// can follow one another in a block.
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
    // Weights are read once: non-temporal loads keep them out of the caches,
    // but only where a row's chunk is whole 128-byte lines; otherwise the line
    // that two consecutive chunks share would be fetched twice.
    constexpr bool kStream = (kCG * kGB) % 128 == 0;
    static_assert(kWRow <= WROW, "tile LDS too small for the format");
    uint8_t* wl = L.wl;

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
    const SxRoles<CG> ro(tid, scales + (int64_t)e * O * G, r0, O, G);

    // ---- weights: a chunk is 64 rows x kPR 16-byte pieces; piece id = tid +
    // 256 i of this thread is (row, part) with each 16 consecutive ids on
    // rows r, r + 4, r + 8, r + 12 and 4 consecutive parts: 64 contiguous
    // bytes per 4 lanes, and their 16-byte LDS stores on 16 disjoint bank
    // quads (the row pitch is 1 mod 4 in 16-byte units).
    constexpr int kPR = kCG * kGB / 16;
    static_assert(kPR % 4 == 0 && (kWRow / 16) % 4 == 1, "conflict-free staging");
    const uint8_t* wsrc[kWPer];  // the piece in chunk 0 (its row's first byte: - 16 part)
    int wdst[kWPer];
    int wpart[kWPer];
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
        const int id = tid + kThreads * i;
        const int g16 = id >> 4, within = id & 15;
        const int rb16 = g16 / (kPR / 4), pq = g16 % (kPR / 4);
        const int row = (rb16 & 3) + 16 * (rb16 >> 2) + 4 * (within >> 2);
        const int part = 4 * pq + (within & 3);
        const int64_t gr = min<int64_t>(r0 + row, O - 1);
        wsrc[i] = pk + gr * G * kGB + 16 * part;
        wdst[i] = row * kWRow + 16 * part;
        wpart[i] = part;
    }
    u32x4_t wv[kWPer];
    SxRegs<CG> sx;
    // full_c: std::true_type for a full chunk (see load_sx), else false_type
    auto load_w = [&](int32_t c0, auto full_c) {
        constexpr bool full = decltype(full_c)::value;
        const int gn = min(kCG, G - c0);
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            // in a short last chunk, pieces past the chunk's bytes re-read the
            // row's first 16 bytes (unused); with G even every piece lies
            // wholly inside or outside
            const int b0 = wpart[i] * 16;
            const uint8_t* rc = wsrc[i] + (int64_t)c0 * kGB;
            const uint8_t* row0 = wsrc[i] - b0;  // always a valid 16 bytes
            if constexpr (W16) {
                const uint8_t* src = full || b0 < gn * kGB ? rc : row0;
                const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(src);
                wv[i] = kStream ? __builtin_nontemporal_load(sp) : *sp;
            } else {
                static_assert(BITS == 3, "int4 groups are always 16-byte aligned");
                const uint8_t* sa = full || b0 < gn * kGB ? rc : row0;
                const uint8_t* sb = full || b0 + 8 < gn * kGB ? rc + 8 : row0;
                const u32x2_t* pa = reinterpret_cast<const u32x2_t*>(sa);
                const u32x2_t* pb = reinterpret_cast<const u32x2_t*>(sb);
                const u32x2_t a = kStream ? __builtin_nontemporal_load(pa) : *pa;
                const u32x2_t b = kStream ? __builtin_nontemporal_load(pb) : *pb;
                wv[i] = u32x4_t{a.x, a.y, b.x, b.y};
            }
        }
    };
    auto is_full = [&](int32_t c0) { return (int64_t)(c0 + kCG) * kGroup <= I; };
    const float* xrow[kTok];
    // loads of chunk c0 into registers, and their stores to LDS, with the
    // clamping of a short last chunk only where it is one (a uniform branch)
    auto load_chunk = [&](int32_t c0) {
        if (is_full(c0)) {
            load_w(c0, std::true_type{});
            load_sx<BITS, CG, XV, true>(sx, ro, c0, xrow, I, G, tid);
        } else {
            load_w(c0, std::false_type{});
            load_sx<BITS, CG, XV, false>(sx, ro, c0, xrow, I, G, tid);
        }
    };
    auto store_chunk = [&](int32_t c0, int nt) {
#pragma unroll
        for (int i = 0; i < kWPer; ++i) *reinterpret_cast<u32x4_t*>(wl + wdst[i]) = wv[i];
        if (is_full(c0))
            store_sx<BITS, CG, true>(sx, ro, c0, nt, L.sl, L.pl, I, G, tid);
        else
            store_sx<BITS, CG, false>(sx, ro, c0, nt, L.sl, L.pl, I, G, tid);
    };

    for (int32_t pb = p0; pb < p1; pb += kTok) {
        const int nt = min(kTok, p1 - pb);
        __syncthreads();  // the previous pass is done with trow/tout and LDS
        pass_tokens(L.trow, L.tout, pb, nt, pair_row, n_x_rows, tid);
        zero_columns<CG>(L.pl, nt, tid);
        __syncthreads();

        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        token_rows(L.trow, X, I, nt, xrow);
        load_chunk(0);
        for (int32_t c0 = 0; c0 < G; c0 += kCG) {
            __syncthreads();  // everyone is done with the previous chunk
            store_chunk(c0, nt);
            __syncthreads();
            // next chunk in flight while this one is multiplied
            if (c0 + kCG < G) load_chunk(c0 + kCG);
            mma_chunk<BITS, CG>(wl, L.pl, L.sl, min(kCG, G - c0), wave, l16, j4, acc);
        }
        store_rows<BITS>(acc, nt, L.tout, r0, O, wave, l16, j4, Y);
    }
}

}  // namespace
}  // namespace qt
