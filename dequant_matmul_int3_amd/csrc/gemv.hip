// int3-g64 (and grouped int4) dequantize-and-multiply on the vector ALUs: one
// or a few input rows against a packed weight matrix, f32 throughout.
//
// Semantics: the "int3-g64 (fmt=5)" pull request page, "Design", Kernel bullet
// (matmul_i3: an exact-f32 path with per-group scale accumulation): for every
// output row, each 64-input group's dot product of codes and inputs is formed
// in f32, multiplied once by the group's f32 scale, and the groups are summed
// in f32.  Grouped int4 follows the same rule with 32-byte nibble groups.
//
// Layout on the GPU (gfx950, wave64):
//  * A block owns RB = WAVES*64/LPR consecutive output rows; LPR lanes share a
//    row, lane q taking groups q, q+LPR, q+2*LPR, ... of the current chunk.
//  * The inputs of the current chunk of groups are staged in LDS as f32, one
//    68-float slot per group (4 floats of padding shift consecutive groups by 4
//    banks, so the 16-byte reads of 16 lanes at a time hit distinct banks).
//  * Every thread issues its input loads, then its weight loads (24 packed
//    bytes and a scale per group), and only then waits to store the inputs to
//    LDS, so the two latencies overlap.
//  * Unpacking is byte-parallel: for low-plane word L (16 codes, code 4b+i in
//    bits 8b+2i..8b+2i+1) and the 16 matching high bits spread one nibble per
//    byte, ((L >> 2i) & 0x03030303) | (high bits at bit 2) gives four u = v+4
//    values, one per byte; v_perm_b32 table lookups turn them into f16 pairs
//    of v (exact), and v_fma_mix_f32 multiplies each by its f32 input with one
//    f32 rounding.  int4 nibbles become f16 pairs by the 1024-bias trick: the
//    f16 word 0x6400 | u is 1024 + u exactly, and one packed f16 subtraction
//    of 1032 leaves v = u - 8.  Four interleaved accumulators per token hide
//    FMA latency.
//  * The LPR partial row sums are combined in a fixed order (DPP steps inside
//    16-lane rows, lane reads across the rows of a wave, then the waves of a
//    row through LDS), so results are deterministic.
//  * Launch shapes: one token uses 16 waves of 128 lanes per row (one group
//    per lane, 8 rows per block, one block per CU at the decode size), so that
//    four waves per SIMD overlap their loads with the other waves' arithmetic;
//    larger tiles use 8 waves of 64 lanes per row.  The inputs of a chunk of
//    GC groups of all T tokens are staged at once.
//  * One f32 token (the decode case) has a kernel of its own: the input
//    vector is copied into LDS once per block by LDS-direct loads
//    (global_load_lds, 16 bytes per lane, no register round trip), and only
//    then are the weight loads issued, so that each wave starts its
//    arithmetic as soon as its own weights arrive.  Issuing the weight loads
//    first was measured slower in every form tried: the input copy then
//    finishes only after the weights, and no wave computes while others
//    still wait.  Blocks loop over 8-row tiles (the next tile's weights in
//    flight while the current one is multiplied), so one launch streams any
//    number of rows with the input staged once per block.
#include <algorithm>

#include "lds_barrier.h"
#include "qt_internal.h"

namespace qt {
namespace {

constexpr int kSlot = kGroup + 4;  // padded LDS floats per group

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int BITS>
struct GroupBits;
template <>
struct GroupBits<3> {
    static constexpr int kBytes = kGroupBytes;
    u32x2_t a, b, c;  // low plane words 0..3, then the high plane
};
template <>
struct GroupBits<4> {
    static constexpr int kBytes = kGroupBytesI4;
    u32x4_t a, b;  // nibble words 0..7: word w holds codes 8w..8w+7
};

// The weights are streamed once per call: non-temporal loads keep them from
// displacing the staged inputs and scales in the caches.
template <int BITS>
__device__ __forceinline__ GroupBits<BITS> load_group(const uint8_t* __restrict__ p) {
    GroupBits<BITS> r;
    if constexpr (BITS == 3) {
        const u32x2_t* q = reinterpret_cast<const u32x2_t*>(p);
        r.a = __builtin_nontemporal_load(q + 0);
        r.b = __builtin_nontemporal_load(q + 1);
        r.c = __builtin_nontemporal_load(q + 2);
    } else {
        const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
        r.a = __builtin_nontemporal_load(q + 0);
        r.b = __builtin_nontemporal_load(q + 1);
    }
    return r;
}

// Spread 16 high-plane bits (bit m = code m of a 16-code quarter) so that the
// bit of code 4b+i lands at bit 2+i of byte b.
__device__ __forceinline__ uint32_t spread_hi(uint32_t h16) {
    uint32_t t = (h16 | (h16 << 8)) & 0x00FF00FFu;
    t = (t | (t << 4)) & 0x0F0F0F0Fu;
    return t << 2;
}

// acc[t][i] += v(code 16k+4b+i) * x_t[16k+4b+i] over b, i for one quarter k,
// for the first NT of T tokens.  u = v + 4 is assembled one code per byte; a
// byte-permute table lookup maps every u to the high byte of the f16 encoding
// of v (whose low byte is zero for v in [-4, 3]) and two more permutes place
// the codes as f16 pairs.  v_fma_mix_f32 then multiplies each f16 code (exact)
// by the f32 input with a single f32 rounding, as an f32 fused multiply-add.
template <int T, int NT>
__device__ __forceinline__ void quarter_fma(uint32_t L, uint32_t sp4, const float* const* xq,
                                            int k, float (&acc)[T][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u4 = ((L >> (2 * i)) & 0x03030303u) | ((sp4 >> i) & 0x04040404u);
        // f16(v) high bytes: u = 0..3 -> c4 c2 c0 bc, u = 4..7 -> 00 3c 40 42
        const uint32_t hb = __builtin_amdgcn_perm(0x42403C00u, 0xBCC0C2C4u, u4);
        const half2_t p01 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(hb, hb, 0x010C000Cu));
        const half2_t p23 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(hb, hb, 0x030C020Cu));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float* x = xq[t] + 16 * k + i;
            acc[t][i] = __builtin_fmaf((float)p01.x, x[0], acc[t][i]);
            acc[t][i] = __builtin_fmaf((float)p01.y, x[4], acc[t][i]);
            acc[t][i] = __builtin_fmaf((float)p23.x, x[8], acc[t][i]);
            acc[t][i] = __builtin_fmaf((float)p23.y, x[12], acc[t][i]);
        }
    }
}

// v_and_or_b32: (a & m) | c in one instruction.  gfx950's three-operand
// encoding takes no literal constants, so the compiler splits a constant mask
// and bias into two literal-operand instructions; here they come in registers.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

// acc[t][i] += v(code 8w+i) * x_t[8w+i] + v(code 8w+4+i) * x_t[8w+4+i] for
// one int4 word w (nibble n = code 8w+n, so the two 16-bit halves hold codes
// 8w..8w+3 and 8w+4..8w+7).  A nibble at bits 0..3 of a half or-ed into the
// f16 word 0x6400 (1024, ulp 1) gives 1024 + u; a nibble at bits 4..7 or-ed
// into 0x5400 (64, ulp 1/16) gives 64 + u.  Both are exact, and so is the
// packed f16 subtraction of 1032 or 72 that leaves v = u - 8.
template <int T, int NT>
__device__ __forceinline__ void word_fma_i4(uint32_t W, const float* const* xq, int w,
                                            float (&acc)[T][4]) {
    const uint32_t lo_bias = 0x64006400u, hi_bias = 0x54005400u;
    const half2_t lo_off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t hi_off = {(_Float16)72.0f, (_Float16)72.0f};
    const uint32_t W8 = W >> 8;
    half2_t p[4];
    p[0] = __builtin_bit_cast(half2_t, and_or(W, 0x000F000Fu, lo_bias)) - lo_off;
    p[1] = __builtin_bit_cast(half2_t, and_or(W, 0x00F000F0u, hi_bias)) - hi_off;
    p[2] = __builtin_bit_cast(half2_t, and_or(W8, 0x000F000Fu, lo_bias)) - lo_off;
    p[3] = __builtin_bit_cast(half2_t, and_or(W8, 0x00F000F0u, hi_bias)) - hi_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float* x = xq[t] + 8 * w + i;
            acc[t][i] = __builtin_fmaf((float)p[i].x, x[0], acc[t][i]);
            acc[t][i] = __builtin_fmaf((float)p[i].y, x[4], acc[t][i]);
        }
    }
}

// Dot of one packed group with the first NT staged input groups: adds, per
// token, scale * sum_j v_j x_j into rowacc[t].
template <int T, int NT, int BITS>
__device__ __forceinline__ void group_dot(const GroupBits<BITS>& gb, float scale,
                                          const float* const* xg, float (&rowacc)[T]) {
    float acc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;
    if constexpr (BITS == 3) {
        const uint32_t L[4] = {gb.a.x, gb.a.y, gb.b.x, gb.b.y};
        const uint32_t H[2] = {gb.c.x, gb.c.y};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t h16 = (H[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
            quarter_fma<T, NT>(L[k], spread_hi(h16), xg, k, acc);
        }
    } else {
        const uint32_t Wd[8] = {gb.a.x, gb.a.y, gb.a.z, gb.a.w, gb.b.x, gb.b.y, gb.b.z, gb.b.w};
#pragma unroll
        for (int w = 0; w < 8; ++w) word_fma_i4<T, NT>(Wd[w], xg, w, acc);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float d = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
        rowacc[t] = __builtin_fmaf(scale, d, rowacc[t]);
    }
}

// Dispatch on the number of live tokens of a tile (uniform over the block), so
// that no multiply is spent on tokens that are not there.
template <int T, int BITS>
__device__ __forceinline__ void group_dot_n(int nt, const GroupBits<BITS>& gb, float scale,
                                            const float* const* xg, float (&rowacc)[T]) {
    if constexpr (T == 1) {
        group_dot<T, 1, BITS>(gb, scale, xg, rowacc);
    } else {
        switch (nt) {
            case 1: group_dot<T, 1, BITS>(gb, scale, xg, rowacc); break;
            case 2: if constexpr (T >= 2) group_dot<T, 2, BITS>(gb, scale, xg, rowacc); break;
            case 3: if constexpr (T >= 3) group_dot<T, 3, BITS>(gb, scale, xg, rowacc); break;
            case 4: if constexpr (T >= 4) group_dot<T, 4, BITS>(gb, scale, xg, rowacc); break;
            default: group_dot<T, T, BITS>(gb, scale, xg, rowacc); break;
        }
    }
}

// Inputs of tokens [0, nt) x groups [g0, g0+gn), staged in LDS as
// [T][GC][kSlot] floats.  Columns at or past I read as 0.  load() issues all
// of a thread's global loads without any branch (out-of-range pieces load a
// valid address and are replaced by zero), so they are all in flight at once;
// store() writes them to LDS.  Callers issue the weight loads in between.
// BF16: inputs are bf16 bit patterns, widened exactly.  VEC: rows allow 16-byte
// (f32) or 8-byte (bf16) loads of 4 columns, I % 4 == 0.
template <int T, int GC, int NTHR, bool BF16, bool VEC>
struct InputStage {
    static constexpr int QUADS = GC * (kGroup / 4);  // 4-column pieces per token
    static constexpr int QPT = (QUADS + NTHR - 1) / NTHR;
    uint4 raw_[T][QPT];  // loaded bits (f32, or bf16 pairs in x, y)
    bool ok_[T][QPT];

    __device__ __forceinline__ void load(const void* __restrict__ X, int64_t row0, int nt,
                                         int64_t I, int64_t g0, int gn) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t row = row0 + (t < nt ? t : 0);
#pragma unroll
            for (int j = 0; j < QPT; ++j) {
                const int qd = tid + j * NTHR;
                const int gl = qd >> 4;
                const int64_t col = (g0 + gl) * kGroup + (qd & 15) * 4;
                const bool live = t < nt && qd < QUADS && gl < gn;
                if constexpr (VEC) {
                    // raw data stay untouched until store(): computing on them
                    // here would make the wave wait for each load in turn
                    const bool ok = live && col < I;
                    const int64_t c = ok ? col : 0;
                    ok_[t][j] = ok;
                    if constexpr (BF16) {
                        const uint2 w = *reinterpret_cast<const uint2*>(
                            reinterpret_cast<const uint16_t*>(X) + row * I + c);
                        raw_[t][j] = make_uint4(w.x, w.y, 0u, 0u);
                    } else {
                        const uint4 w = *reinterpret_cast<const uint4*>(
                            reinterpret_cast<const float*>(X) + row * I + c);
                        raw_[t][j] = w;
                    }
                } else {
                    float e[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bool ok = live && col + q < I;
                        const int64_t c = ok ? col + q : 0;
                        float f;
                        if constexpr (BF16)
                            f = __uint_as_float(
                                (uint32_t)(reinterpret_cast<const uint16_t*>(X)[row * I + c])
                                << 16);
                        else
                            f = reinterpret_cast<const float*>(X)[row * I + c];
                        e[q] = ok ? f : 0.0f;
                    }
                    ok_[t][j] = true;
                    raw_[t][j] = make_uint4(__float_as_uint(e[0]), __float_as_uint(e[1]),
                                            __float_as_uint(e[2]), __float_as_uint(e[3]));
                }
            }
        }
    }

    __device__ __forceinline__ void store(int nt, float* xs) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int j = 0; j < QPT; ++j) {
                const int qd = tid + j * NTHR;
                if (t < nt && qd < QUADS) {
                    float* dst = xs + (t * GC + (qd >> 4)) * kSlot + (qd & 15) * 4;
                    const uint4 w = raw_[t][j];
                    float4 f;
                    if constexpr (VEC && BF16)
                        f = make_float4(__uint_as_float(w.x << 16),
                                        __uint_as_float(w.x & 0xFFFF0000u),
                                        __uint_as_float(w.y << 16),
                                        __uint_as_float(w.y & 0xFFFF0000u));
                    else
                        f = make_float4(__uint_as_float(w.x), __uint_as_float(w.y),
                                        __uint_as_float(w.z), __uint_as_float(w.w));
                    if (!ok_[t][j]) f = make_float4(0.f, 0.f, 0.f, 0.f);
                    *reinterpret_cast<float4*>(dst) = f;
                }
            }
    }
};

// Sum over aligned groups of WL lanes (WL = 16, 32 or 64), valid in the
// first lane of each group, in a fixed order: pairs and quads by quad
// permutes, then rotations by 4 and 8 inside each 16-lane row, then the row
// sums read from lanes 0, 16, 32, 48.
template <int DPP>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), DPP, 0xF, 0xF, false));
}

template <int WL>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(WL == 16 || WL == 32 || WL == 64, "16, 32 or 64 lanes");
    v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x124>(v);  // row_ror 4
    v += dpp_f<0x128>(v);  // row_ror 8
    if constexpr (WL == 16) {
        return v;
    } else {
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
        if constexpr (WL == 32)
            return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
        else
            return (r0 + r1) + (r2 + r3);
    }
}

// Rows [r0, r0+RB) of one matrix against tokens tok0 .. tok0+ntok-1 (the
// input and output rows), T tokens per pass over the weights.
template <int LPR, int WAVES, int T, int GC, bool BF16, bool VEC, int BITS>
__device__ void gemv_rows(const uint8_t* __restrict__ packed, const float* __restrict__ scales,
                          int64_t O, int64_t I, int64_t G, const void* __restrict__ X,
                          int64_t tok0, int ntok, float* __restrict__ Y, int64_t r0, float* lds) {
    constexpr int NTHR = WAVES * 64;
    constexpr int NG = (GC + LPR - 1) / LPR;  // groups per lane per chunk
    static_assert(GC >= LPR, "each lane needs at least one group per chunk");
    float* xs = lds;

    const int q = threadIdx.x % LPR;
    const int64_t r = r0 + threadIdx.x / LPR;
    const bool row_ok = r < O;

    for (int tt = 0; tt < ntok; tt += T) {
        const int nt = min(T, ntok - tt);
        float rowacc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) rowacc[t] = 0.0f;

        for (int64_t g0 = 0; g0 < G; g0 += GC) {
            const int gn = (int)min<int64_t>(GC, G - g0);
            if (tt > 0 || g0 > 0) __syncthreads();  // earlier readers are done with LDS
            InputStage<T, GC, NTHR, BF16, VEC> stage;
            stage.load(X, tok0 + tt, nt, I, g0, gn);
            // weight loads, branch-free: idle lanes load group 0 of the block's
            // first row (always valid) and are not used.  The compiler issues
            // them after the staging barrier below (their uses sit in the
            // branch after it); issuing them before it, so that they were in
            // flight during the staging, measured slower: 5.3 against 4.75 us
            // per decode launch.
            GroupBits<BITS> gb[NG];
            float sc[NG];
#pragma unroll
            for (int m = 0; m < NG; ++m) {
                const int gl = q + m * LPR;
                const bool ok = row_ok && gl < gn;
                const int64_t gi = ok ? r * G + g0 + gl : r0 * G;
                gb[m] = load_group<BITS>(packed + gi * GroupBits<BITS>::kBytes);
                sc[m] = scales[gi];
            }
            stage.store(nt, xs);
            __syncthreads();
#pragma unroll
            for (int m = 0; m < NG; ++m) {
                const int gl = q + m * LPR;
                if (row_ok && gl < gn) {
                    const float* xg[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) xg[t] = xs + (t * GC + gl) * kSlot;
                    group_dot_n<T, BITS>(nt, gb[m], sc[m], xg, rowacc);
                }
            }
        }
        // combine the LPR partial sums of each row in a fixed order: DPP
        // steps inside each 16-lane row, the rows of a wave through lane
        // reads, then (rows wider than a wave) the per-wave sums in wave order
        // through LDS
        constexpr int WL = LPR < 64 ? LPR : 64;
#pragma unroll
        for (int t = 0; t < T; ++t) rowacc[t] = lane_group_sum<WL>(rowacc[t]);
        if constexpr (LPR > 64) {
            constexpr int PARTS = LPR / 64;
            __shared__ float part[WAVES * T];  // [row in block][part][T]
            const int rb = threadIdx.x / LPR, pw = q / 64;
            if ((q & 63) == 0) {
#pragma unroll
                for (int t = 0; t < T; ++t) part[(rb * PARTS + pw) * T + t] = rowacc[t];
            }
            __syncthreads();
            if (q == 0) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    float a = part[(rb * PARTS) * T + t];
#pragma unroll
                    for (int w = 1; w < PARTS; ++w) a += part[(rb * PARTS + w) * T + t];
                    rowacc[t] = a;
                }
            }
        }
        if (row_ok && q == 0) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (t < nt) Y[(tok0 + tt + t) * O + r] = rowacc[t];
        }
    }
}

template <int T, int GC>
constexpr size_t lds_bytes() {
    return (size_t)T * GC * kSlot * sizeof(float);
}

// ---------------------------------------------------------------- kernels
constexpr int kMaxTok = 16;  // token rows per launch chunk of the batch kernel

template <int LPR, int WAVES, int T, int GC, bool BF16, bool VEC, int BITS>
__global__ __launch_bounds__(WAVES * 64) void gemv_batch_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int64_t I,
    int64_t G, const void* __restrict__ X, int64_t tok0, int ntok, float* __restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int RB = WAVES * 64 / LPR;
    gemv_rows<LPR, WAVES, T, GC, BF16, VEC, BITS>(packed, scales, O, I, G, X, tok0, ntok, Y,
                                              (int64_t)blockIdx.x * RB, lds);
}

}  // namespace

// Decode and small batches.  LPR/WAVES chosen so that O/RB blocks cover the
// chip; tokens in tiles of T per pass over the weights.
template <int LPR, int WAVES, int T, int GC, bool BF16, bool VEC, int BITS>
static hipError_t run_batch(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                            const void* X, int64_t ntok, float* Y, hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    constexpr int RB = WAVES * 64 / LPR;
    const int64_t blocks = (O + RB - 1) / RB;
    for (int64_t t0 = 0; t0 < ntok; t0 += kMaxTok) {
        const int n = (int)std::min<int64_t>(kMaxTok, ntok - t0);
        hipLaunchKernelGGL((gemv_batch_kernel<LPR, WAVES, T, GC, BF16, VEC, BITS>),
                           dim3((unsigned)blocks), dim3(WAVES * 64), (lds_bytes<T, GC>()), s, packed,
                           scales, O, I, G, X, t0, n, Y);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------- decode kernel
// One f32 input vector, lane q of a row taking groups q, q + 128, ... (at
// most kDecMaxG groups, all staged at once).  LDS layout of x: 16-byte piece p
// (columns 4p .. 4p+3) at byte (p / 64) * kDecChunk + (p % 64) * 16, i.e. four
// groups per 1024-byte run, each run padded by 16 bytes.
constexpr int kDecRows = 8;       // rows per tile
constexpr int kDecMaxG = 256;     // groups per row the decode kernel stages
constexpr int kDecChunk = 1040;   // LDS bytes per 64 pieces (4 groups)

__device__ __forceinline__ const float* dec_group(const float* xs, int64_t g) {
    return reinterpret_cast<const float*>(reinterpret_cast<const char*>(xs) + (g >> 2) * kDecChunk +
                                          (g & 3) * 256);
}

// NG: groups per lane (G <= 128 NG).  LOOP: blocks take several 8-row tiles
// (the next tile's weights in flight while the current one is multiplied);
// otherwise each block multiplies one tile.
template <int BITS, int NG, bool LOOP>
__global__ __launch_bounds__(1024) void gemv_decode_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int O, int I,
    int G, const float* __restrict__ x, float* __restrict__ y, int ntiles) {
    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(1))) void glob_void;
    extern __shared__ __attribute__((aligned(16))) float xs[];
    __shared__ float part[2][16];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int q = tid & 127;
    const int rl = tid >> 7;

    // ---- x into LDS: wave w copies runs w, w + 16, ...; pieces past I are
    // zeroed (I % 4 == 0, so a piece lies wholly inside or outside x)
    const int nruns = (G + 3) / 4;
    for (int c = w; c < nruns; c += 16) {
        const int pc = c * 64 + lane;  // piece: columns 4 pc .. 4 pc + 3
        char* base = reinterpret_cast<char*>(xs) + c * kDecChunk;  // wave-uniform
        if (4 * pc < I)
            __builtin_amdgcn_global_load_lds((const glob_void*)(x + 4 * pc), (lds_void*)base, 16, 0,
                                             0);
        else if (pc < 16 * G)
            *reinterpret_cast<float4*>(base + 16 * lane) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    const float* xg[NG][1];
#pragma unroll
    for (int m = 0; m < NG; ++m) xg[m][0] = dec_group(xs, q + 128 * m < G ? q + 128 * m : 0);
    // one group per lane: its 64 inputs are read into registers once and serve
    // every tile of the block (read after the first tile's weight loads are
    // issued, so the LDS reads do not wait for the weights; reading them inside
    // the arithmetic instead measured 0.4 us slower per decode launch)
    float xr[NG == 1 ? kGroup : 1];
    const float* xrp[1] = {xr};
    auto read_x = [&]() {
        if constexpr (NG == 1) {
#pragma unroll
            for (int k = 0; k < kGroup / 4; ++k) {
                const float4 v = reinterpret_cast<const float4*>(xg[0][0])[k];
                xr[4 * k] = v.x;
                xr[4 * k + 1] = v.y;
                xr[4 * k + 2] = v.z;
                xr[4 * k + 3] = v.w;
            }
        }
    };

    // ---- lanes past G and rows past O load nothing and skip the arithmetic
    auto load_tile = [&](int tile, GroupBits<BITS> (&gb)[NG], float (&sc)[NG]) {
        const int r = tile * kDecRows + rl;
#pragma unroll
        for (int m = 0; m < NG; ++m) {
            const int g = q + 128 * m;
            if (r < O && g < G) {
                const int64_t gi = (int64_t)r * G + g;
                gb[m] = load_group<BITS>(packed + gi * GroupBits<BITS>::kBytes);
                sc[m] = scales[gi];
            }
        }
    };
    auto mul_tile = [&](int tile, int it, const GroupBits<BITS> (&gb)[NG], const float (&sc)[NG]) {
        const int r = tile * kDecRows + rl;
        float rowacc[1] = {0.0f};
        if constexpr (NG == 1) {
            if (r < O && q < G) group_dot<1, 1, BITS>(gb[0], sc[0], xrp, rowacc);
        } else {
#pragma unroll
            for (int m = 0; m < NG; ++m)
                if (r < O && q + 128 * m < G) group_dot<1, 1, BITS>(gb[m], sc[m], xg[m], rowacc);
        }
        const float acc = lane_group_sum<64>(rowacc[0]);
        // the two waves of a row in a fixed order; part is double-buffered by
        // tile parity, so one barrier per tile suffices (an LDS-only one: the
        // next tiles' weight loads stay in flight across it)
        if (lane == 0) part[it & 1][w] = acc;
        lds_barrier();
        if (q == 0 && r < O) y[r] = part[it & 1][w] + part[it & 1][w + 1];
    };
    GroupBits<BITS> cur[NG];
    float cs[NG];
    if constexpr (!LOOP) {
        load_tile(blockIdx.x, cur, cs);
        read_x();
        mul_tile(blockIdx.x, 0, cur, cs);
    } else {
        // a ring of four tiles' weights: the next three in flight while one
        // is multiplied.  The loop is unrolled by the ring's size, so every
        // step names its buffers statically: rotating them by copies instead
        // made each copy of a register still being loaded wait for that load,
        // and the loop head waited for every load in flight.
        //   Every step issues the same loads, so the compiler can tell which
        // are still in flight and waits only for the tile it multiplies:
        // lanes past G and rows past O load a valid group (unused), and
        // steps past the block's last tile load group 0 in every lane
        // (unused; one line, which stays cached).
        GroupBits<BITS> ring[4][NG];
        float rs[4][NG];
        const int step = gridDim.x;
        int tile = blockIdx.x;
        const int last = tile + (ntiles - 1 - tile) / step * step;  // this block's last tile
        const int64_t tile_groups = (int64_t)kDecRows * G;          // groups of one tile
        int64_t gi0[NG];  // group index of this lane's group in the block's first tile
#pragma unroll
        for (int m = 0; m < NG; ++m)
            gi0[m] = (int64_t)min(tile * kDecRows + rl, O - 1) * G + min(q + 128 * m, G - 1);
        auto load_ring = [&](int t, GroupBits<BITS> (&gb)[NG], float (&sc)[NG]) {
            // rows of tile t past O: the block's first tile's row (unused)
            const int64_t dt = t * kDecRows + rl < O ? (int64_t)(t - blockIdx.x) * tile_groups : 0;
#pragma unroll
            for (int m = 0; m < NG; ++m) {
                const int64_t gi = t <= last ? gi0[m] + dt : 0;
                gb[m] = load_group<BITS>(packed + gi * GroupBits<BITS>::kBytes);
                sc[m] = scales[gi];
            }
        };
        load_ring(tile, ring[0], rs[0]);
        load_ring(tile + step, ring[1], rs[1]);
        load_ring(tile + 2 * step, ring[2], rs[2]);
        read_x();
        for (int it = 0; tile < ntiles;) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                load_ring(tile + 3 * step, ring[(k + 3) % 4], rs[(k + 3) % 4]);
                if (tile < ntiles) mul_tile(tile, it, ring[k], rs[k]);  // uniform
                tile += step;
                ++it;
            }
        }
    }
}

// One 8-row tile per block, G <= 128: the plainest form of the decode kernel
// (x copied into LDS, then each lane's weight loads and its group's dot
// product read straight from LDS), which measured fastest for one tile.
template <int BITS>
__global__ __launch_bounds__(1024) void gemv_decode1_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int O, int I, int G,
    const float* __restrict__ x, float* __restrict__ y) {
    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(1))) void glob_void;
    extern __shared__ __attribute__((aligned(16))) float xs[];
    __shared__ float part[16];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int q = tid & 127;
    const int r = blockIdx.x * kDecRows + (tid >> 7);
    const int nruns = (G + 3) / 4;
    for (int c = w; c < nruns; c += 16) {
        const int pc = c * 64 + lane;
        char* base = reinterpret_cast<char*>(xs) + c * kDecChunk;
        if (4 * pc < I)
            __builtin_amdgcn_global_load_lds((const glob_void*)(x + 4 * pc), (lds_void*)base, 16, 0,
                                             0);
        else if (pc < 16 * G)
            *reinterpret_cast<float4*>(base + 16 * lane) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    float acc = 0.0f;
    if (q < G && r < O) {
        const int64_t gi = (int64_t)r * G + q;
        const GroupBits<BITS> gb = load_group<BITS>(packed + gi * GroupBits<BITS>::kBytes);
        const float sc = scales[gi];
        const float* xg[1] = {dec_group(xs, q)};
        float ra[1] = {0.0f};
        group_dot<1, 1, BITS>(gb, sc, xg, ra);
        acc = ra[0];
    }
    acc = lane_group_sum<64>(acc);
    if (lane == 0) part[w] = acc;
    __syncthreads();
    if (q == 0 && r < O) y[r] = part[w] + part[w + 1];
}

template <int BITS>
static hipError_t run_decode(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                             const float* x, float* y, hipStream_t s) {
    const int G = (int)((I + kGroup - 1) / kGroup);
    const int ntiles = (int)((O + kDecRows - 1) / kDecRows);
    // one tile per block up to 512 tiles (two one-tile blocks fit on each of
    // the 256 CUs); more tiles loop, one block per CU (the looping kernel's
    // registers leave room for one 1024-thread block per CU)
    const int blocks = std::min(ntiles, 512);
    const size_t lds = (size_t)((G + 3) / 4) * kDecChunk;
    const dim3 grid((unsigned)blocks), block(1024);
    const dim3 loop_grid((unsigned)std::min(ntiles, 256));
#define QT_DEC(NG, LOOP)                                                                      \
    hipLaunchKernelGGL((gemv_decode_kernel<BITS, NG, LOOP>), LOOP ? loop_grid : grid, block, \
                       lds, s, packed, scales, (int)O, (int)I, G, x, y, ntiles)
    if (G <= 128) {
        if (ntiles <= blocks)
            hipLaunchKernelGGL((gemv_decode1_kernel<BITS>), grid, block, lds, s, packed, scales,
                               (int)O, (int)I, G, x, y);
        else
            QT_DEC(1, true);
    } else {
        if (ntiles <= blocks) QT_DEC(2, false);
        else QT_DEC(2, true);
    }
#undef QT_DEC
    return hipGetLastError();
}

template <bool BF16, bool VEC, int BITS>
static hipError_t batch_dispatch(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                                 const void* X, int64_t ntok, float* Y, hipStream_t s) {
    if (ntok == 1) return run_batch<128, 16, 1, 128, BF16, VEC, BITS>(packed, scales, O, I, X, 1, Y, s);
    if (ntok == 2) return run_batch<128, 16, 2, 128, BF16, VEC, BITS>(packed, scales, O, I, X, 2, Y, s);
    if (ntok <= 4)
        return run_batch<64, 8, 4, 128, BF16, VEC, BITS>(packed, scales, O, I, X, ntok, Y, s);
    return run_batch<64, 8, 8, 64, BF16, VEC, BITS>(packed, scales, O, I, X, ntok, Y, s);
}

template <int BITS>
static hipError_t gemv_bits(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                            const void* X, bool bf16, int64_t ntok, float* Y, hipStream_t s) {
    // 16-byte (f32) or 8-byte (bf16) input loads need aligned rows
    const uintptr_t al = bf16 ? 8 : 16;
    const bool vec = (I % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & (al - 1)) == 0);
    // the decode kernel indexes rows and columns in 32 bits
    if (!bf16 && vec && ntok == 1 && (I + kGroup - 1) / kGroup <= kDecMaxG && O <= (1 << 28))
        return run_decode<BITS>(packed, scales, O, I, static_cast<const float*>(X), Y, s);
    if (bf16)
        return vec ? batch_dispatch<true, true, BITS>(packed, scales, O, I, X, ntok, Y, s)
                   : batch_dispatch<true, false, BITS>(packed, scales, O, I, X, ntok, Y, s);
    return vec ? batch_dispatch<false, true, BITS>(packed, scales, O, I, X, ntok, Y, s)
               : batch_dispatch<false, false, BITS>(packed, scales, O, I, X, ntok, Y, s);
}

hipError_t launch_gemv_batch(const uint8_t* packed, const float* scales, int64_t O,
                             int64_t I, const void* X, bool bf16, int64_t ntok, float* Y,
                             hipStream_t s, int bits) {
    if (bits == 3) return gemv_bits<3>(packed, scales, O, I, X, bf16, ntok, Y, s);
    if (bits == 4) return gemv_bits<4>(packed, scales, O, I, X, bf16, ntok, Y, s);
    return hipErrorInvalidValue;
}

}  // namespace qt
