// int3-g64 dequantize-and-multiply on the vector ALUs: one or a few input rows
// against a packed weight matrix, f32 throughout.
//
// Semantics: the "int3-g64 (fmt=5)" pull request page, "Design", Kernel bullet
// (matmul_i3: an exact-f32 path with per-group scale accumulation): for every
// output row, each 64-input group's dot product of codes and inputs is formed
// in f32, multiplied once by the group's f32 scale, and the groups are summed
// in f32.
//
// Layout on the GPU (gfx950, wave64):
//  * A block owns RB = WAVES*64/LPR consecutive output rows; LPR lanes share a
//    row, lane q taking groups q, q+LPR, q+2*LPR, ... of the current chunk.
//  * The inputs of the current chunk of groups are staged in LDS as f32, one
//    68-float slot per group (4 floats of padding shift consecutive groups by 4
//    banks).  All rows of a wave read the same addresses, which LDS broadcasts.
//  * A lane fetches its groups' 24 packed bytes (three 8-byte loads) and
//    scales before the chunk's inputs are staged, so the HBM latency overlaps
//    the staging.
//  * Unpacking is byte-parallel: for low-plane word L (16 codes, code 4b+i in
//    bits 8b+2i..8b+2i+1) and the 16 matching high bits spread one nibble per
//    byte, ((L >> 2i) & 0x03030303) | (high bits at bit 2) gives four u = v+4
//    values, one per byte; one v_perm_b32 table lookup maps them to the signed
//    bytes v, which convert to f32 exactly.  Products v*x are formed with
//    fused multiply-adds into four interleaved accumulators per token (hiding
//    FMA latency); the LPR partial row sums are combined by a fixed xor
//    butterfly, so results are deterministic.
#include <algorithm>

#include "qt_internal.h"

namespace qt {
namespace {

constexpr int kSlot = kGroup + 4;  // padded LDS floats per group

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

struct GroupBits {
    u32x2_t a, b, c;  // low plane words 0..3, then the high plane
};

// The weights are streamed once per call: non-temporal loads keep them from
// displacing the staged inputs and scales in the caches.
__device__ __forceinline__ GroupBits load_group(const uint8_t* __restrict__ p) {
    const u32x2_t* q = reinterpret_cast<const u32x2_t*>(p);
    GroupBits r;
    r.a = __builtin_nontemporal_load(q + 0);
    r.b = __builtin_nontemporal_load(q + 1);
    r.c = __builtin_nontemporal_load(q + 2);
    return r;
}

// Spread 16 high-plane bits (bit m = code m of a 16-code quarter) so that the
// bit of code 4b+i lands at bit 2+i of byte b.
__device__ __forceinline__ uint32_t spread_hi(uint32_t h16) {
    uint32_t t = (h16 | (h16 << 8)) & 0x00FF00FFu;
    t = (t | (t << 4)) & 0x0F0F0F0Fu;
    return t << 2;
}

// acc[t][i] += v(code 16k+4b+i) * x_t[16k+4b+i] over b, i for one quarter k.
// u = v + 4 is assembled one code per byte, a byte-permute table lookup turns
// every u into the signed byte v, and each byte is converted to f32 exactly.
template <int T>
__device__ __forceinline__ void quarter_fma(uint32_t L, uint32_t sp4, const float* const* xq,
                                            int k, float (&acc)[T][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u4 = ((L >> (2 * i)) & 0x03030303u) | ((sp4 >> i) & 0x04040404u);
        // table: u = 0..3 -> fc fd fe ff, u = 4..7 -> 00 01 02 03
        const uint32_t v4 = __builtin_amdgcn_perm(0x03020100u, 0xFFFEFDFCu, u4);
        const float v0 = (float)(int8_t)(uint8_t)v4;
        const float v1 = (float)(int8_t)(uint8_t)(v4 >> 8);
        const float v2 = (float)(int8_t)(uint8_t)(v4 >> 16);
        const float v3 = (float)(int8_t)(uint8_t)(v4 >> 24);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float* x = xq[t] + 16 * k + i;
            acc[t][i] = __builtin_fmaf(v0, x[0], acc[t][i]);
            acc[t][i] = __builtin_fmaf(v1, x[4], acc[t][i]);
            acc[t][i] = __builtin_fmaf(v2, x[8], acc[t][i]);
            acc[t][i] = __builtin_fmaf(v3, x[12], acc[t][i]);
        }
    }
}

// Dot of one packed group with T staged input groups: adds, per token,
// scale * sum_j v_j x_j into rowacc[t].
template <int T>
__device__ __forceinline__ void group_dot(const GroupBits& gb, float scale,
                                          const float* const* xg, float (&rowacc)[T]) {
    float acc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;
    const uint32_t L[4] = {gb.a.x, gb.a.y, gb.b.x, gb.b.y};
    const uint32_t H[2] = {gb.c.x, gb.c.y};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t h16 = (H[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
        quarter_fma<T>(L[k], spread_hi(h16), xg, k, acc);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float d = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
        rowacc[t] = __builtin_fmaf(scale, d, rowacc[t]);
    }
}

// Stage tokens [tok0, tok0+nt) x groups [g0, g0+gn) of the inputs into LDS
// as [T][GC][kSlot] floats.  Columns at or past I read as 0.
template <int T, int GC, int NTHR>
__device__ __forceinline__ void stage_inputs(const void* __restrict__ X, bool bf16,
                                             const int32_t* rows, int nt, int64_t I,
                                             int64_t g0, int gn, float* xs) {
    const int tid = threadIdx.x;
    // 4 columns per thread step
    const int quads = gn * (kGroup / 4);
    for (int t = 0; t < nt; ++t) {
        const int64_t row = rows[t];
        for (int qd = tid; qd < quads; qd += NTHR) {
            const int gl = qd >> 4;
            const int j = (qd & 15) * 4;
            const int64_t col = (g0 + gl) * kGroup + j;
            float v[4];
            if (bf16) {
                const uint16_t* xr = reinterpret_cast<const uint16_t*>(X) + row * I;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = col + e < I ? __uint_as_float((uint32_t)xr[col + e] << 16) : 0.0f;
            } else {
                const float* xr = reinterpret_cast<const float*>(X) + row * I;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = col + e < I ? xr[col + e] : 0.0f;
            }
            float* dst = xs + (t * GC + gl) * kSlot + j;
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    __syncthreads();
}

// Rows [r0, r0+RB) of one matrix against up to T staged tokens at a time.
// rows_of_tok: input row of each token; out_of_tok: output row (times O) of
// each token.  Tokens are processed in tiles of T.
template <int LPR, int WAVES, int T>
__device__ void gemv_rows(const uint8_t* __restrict__ packed, const float* __restrict__ scales,
                          int64_t O, int64_t I, int64_t G, const void* __restrict__ X, bool bf16,
                          const int32_t* tok_rows, const int32_t* tok_outs, int ntok,
                          float* __restrict__ Y, int64_t r0, float* lds) {
    constexpr int NTHR = WAVES * 64;
    constexpr int GC = 128 / T;          // groups per chunk
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
            // issue this lane's weight loads before staging the inputs
            GroupBits gb[NG];
            float sc[NG];
#pragma unroll
            for (int m = 0; m < NG; ++m) {
                const int gl = q + m * LPR;
                if (row_ok && gl < gn) {
                    const int64_t gi = r * G + g0 + gl;
                    gb[m] = load_group(packed + gi * kGroupBytes);
                    sc[m] = scales[gi];
                } else {
                    gb[m] = GroupBits{};
                    sc[m] = 0.0f;
                }
            }
            __syncthreads();  // previous chunk's readers are done with LDS
            stage_inputs<T, GC, NTHR>(X, bf16, tok_rows + tt, nt, I, g0, gn, xs);
#pragma unroll
            for (int m = 0; m < NG; ++m) {
                const int gl = q + m * LPR;
                if (row_ok && gl < gn) {
                    const float* xg[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) xg[t] = xs + (t * GC + gl) * kSlot;
                    group_dot<T>(gb[m], sc[m], xg, rowacc);
                }
            }
        }
        // combine the LPR partial sums of each row (fixed butterfly)
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) rowacc[t] += __shfl_xor(rowacc[t], m, LPR);
        }
        if (row_ok && q == 0) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (t < nt && tok_outs[tt + t] >= 0)
                    Y[(int64_t)tok_outs[tt + t] * O + r] = rowacc[t];
        }
    }
}

template <int T>
constexpr size_t lds_bytes() {
    return (size_t)T * (128 / T) * kSlot * sizeof(float);
}

// ---------------------------------------------------------------- kernels
constexpr int kMaxTok = 16;  // token rows per launch chunk of the batch kernel

template <int LPR, int WAVES, int T>
__global__ __launch_bounds__(WAVES * 64) void gemv_batch_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int64_t I,
    int64_t G, const void* __restrict__ X, int bf16, int64_t tok0, int ntok,
    float* __restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ int32_t rows[kMaxTok];
    if (threadIdx.x < kMaxTok) rows[threadIdx.x] = (int32_t)(tok0 + threadIdx.x);
    __syncthreads();
    constexpr int RB = WAVES * 64 / LPR;
    gemv_rows<LPR, WAVES, T>(packed, scales, O, I, G, X, bf16 != 0, rows, rows, ntok, Y,
                             (int64_t)blockIdx.x * RB, lds);
}

// grid: (row blocks, experts).  Pairs of expert e: [off[e], off[e+1]).
template <int LPR, int WAVES, int T>
__global__ __launch_bounds__(WAVES * 64) void gemv_grouped_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int64_t I,
    int64_t G, const float* __restrict__ X, int64_t n_x_rows, const int32_t* __restrict__ pair_row,
    const int32_t* __restrict__ off, int32_t E, int32_t P, float* __restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ int32_t rows[kMaxTok];
    __shared__ int32_t outs[kMaxTok];
    const int e = blockIdx.y;
    const int32_t p0 = max(0, min(off[e], P));
    const int32_t p1 = max(p0, min(off[e + 1], P));
    if (p1 == p0) return;  // uniform over the block
    constexpr int RB = WAVES * 64 / LPR;
    const uint8_t* pk = packed + (int64_t)e * O * G * kGroupBytes;
    const float* sc = scales + (int64_t)e * O * G;
    for (int32_t pb = p0; pb < p1; pb += kMaxTok) {
        const int n = min(kMaxTok, p1 - pb);
        __syncthreads();
        if (threadIdx.x < n) {
            const int32_t p = pb + threadIdx.x;
            int32_t xr = pair_row ? pair_row[p] : p;
            // out-of-range rows read row 0 and are not written; the host
            // documents the valid range, this only keeps accesses in bounds
            outs[threadIdx.x] = (xr >= 0 && xr < n_x_rows) ? p : -1;
            rows[threadIdx.x] = (xr >= 0 && xr < n_x_rows) ? xr : 0;
        }
        __syncthreads();
        gemv_rows<LPR, WAVES, T>(pk, sc, O, I, G, X, false, rows, outs, n, Y,
                                 (int64_t)blockIdx.x * RB, lds);
    }
}

}  // namespace

// Decode and small batches.  LPR/WAVES chosen so that O/RB blocks cover the
// chip; tokens in tiles of T per pass over the weights.
template <int LPR, int WAVES, int T>
static hipError_t run_batch(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                            const void* X, bool bf16, int64_t ntok, float* Y, hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    constexpr int RB = WAVES * 64 / LPR;
    const int64_t blocks = (O + RB - 1) / RB;
    for (int64_t t0 = 0; t0 < ntok; t0 += kMaxTok) {
        const int n = (int)std::min<int64_t>(kMaxTok, ntok - t0);
        hipLaunchKernelGGL((gemv_batch_kernel<LPR, WAVES, T>), dim3((unsigned)blocks),
                           dim3(WAVES * 64), lds_bytes<T>(), s, packed, scales, O, I, G, X,
                           (int)bf16, t0, n, Y);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_batch(const uint8_t* packed, const float* scales, int64_t O,
                             int64_t I, const void* X, bool bf16, int64_t ntok, float* Y,
                             hipStream_t s) {
    if (ntok == 1) return run_batch<32, 4, 1>(packed, scales, O, I, X, bf16, 1, Y, s);
    if (ntok == 2) return run_batch<32, 4, 2>(packed, scales, O, I, X, bf16, 2, Y, s);
    if (ntok <= 4) return run_batch<16, 4, 4>(packed, scales, O, I, X, bf16, ntok, Y, s);
    return run_batch<16, 4, 8>(packed, scales, O, I, X, bf16, ntok, Y, s);
}

hipError_t launch_gemv_grouped(const uint8_t* packed, const float* scales, int32_t E,
                               int64_t O, int64_t I, const float* X, int64_t n_x_rows,
                               const int32_t* pair_row, const int32_t* expert_offsets,
                               int32_t P, float* Y, hipStream_t s) {
    constexpr int LPR = 16, WAVES = 4, T = 4;
    constexpr int RB = WAVES * 64 / LPR;
    const int64_t G = (I + kGroup - 1) / kGroup;
    const int64_t rb = (O + RB - 1) / RB;
    hipLaunchKernelGGL((gemv_grouped_kernel<LPR, WAVES, T>), dim3((unsigned)rb, (unsigned)E),
                       dim3(WAVES * 64), lds_bytes<T>(), s, packed, scales, O, I, G, X,
                       n_x_rows, pair_row, expert_offsets, E, P, Y);
    return hipGetLastError();
}

}  // namespace qt
