// A mixture-of-experts expert layer as a sequence of launches on the
// caller's stream (the pull request page's MoE decode setting: every routed
// expert's weights read once per step; its per-projection ablation names
// gate_proj, up_proj and down_proj, each at int3-g64 or grouped int4):
//
//  0. routing (one block): per token the k largest logits (equal logits:
//     lower expert first), combine weights a softmax over them; the
//     (expert, token) pairs sorted by expert, then token.
//  1. gate and up: the grouped matrix-core tile (grouped_tile.h) over
//     (64-row block, expert, projection), g and u for every pair.
//  2. h = silu(g) * u for every pair and row.
//  3. down: the grouped launch on h (a pair's row of h is its input).
//  4. out[t] = sum_j w_tj y_{pair(t, j)} in j order.
// Every output is written once by one thread, in a fixed order, so the
// results do not depend on scheduling.
#include "grouped_tile.h"

namespace qt {
namespace {

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 512;  // routing keeps a token's keys in registers (32 per lane)

struct MoeArgs {
    const float* X;  // [T x D]
    const float* logits;  // [T x E]
    int32_t T, D, F, E, k;
    const uint8_t* gp;
    const float* gs;
    const uint8_t* up;
    const float* us;
    const uint8_t* dp;
    const float* ds;
    int32_t gbits, ubits, dbits;
    float* out;  // [T x D]
    // workspace
    int32_t* sel;    // [T k] expert of (t, j)
    float* wgt;      // [T k] combine weight of (t, j)
    int32_t* slot;   // [T k] pair index of (t, j)
    int32_t* prow;   // [P] token of pair p
    int32_t* offs;   // [E + 1]
    float* Yg;       // [P x F]
    float* Yu;       // [P x F]
    float* H;        // [P x F] silu(g) * u
    float* Yd;       // [P x D]
};

// Stage 0, one block of NT threads: 16 lanes per token, NT / 16 tokens per
// pass (NT falls as the experts per lane, and so the registers, grow).  Each pick is the largest key below the previous pick
// (keys order (logit, expert): larger logit first, then lower expert), a
// lane's maximum over its experts, then over the 16 lanes.  Each pair's
// slot is its expert's offset plus the number of earlier tokens that chose
// that expert: per pass a bit per (expert, token of the pass) in LDS, the
// bits below a token counted, plus the expert's total over earlier passes
// (a token picks an expert at most once, so this is deterministic).
constexpr int kRouteMaxTokens = 64;  // tokens per pass at most: two mask words per expert
constexpr int kRouteLdsPairs = 4096;  // packed pairs kept in LDS up to this

// value of lane (l - N) mod 16 of this lane's 16-lane row
template <int N>
__device__ __forceinline__ int row_ror(int v) {
    return __builtin_amdgcn_mov_dpp(v, 0x120 + N, 0xF, 0xF, false);
}

// Routing keys: a total order on (logit, expert) as one 64-bit integer,
// larger logit first, then lower expert index: the logit's bits made
// monotone (-0 folded to +0 first, so equal logits compare equal) above
// 0xFFFF - e.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(0xFFFF - e);
}
__device__ __forceinline__ int key_expert(uint64_t key) {
    return 0xFFFF - (int)(key & 0xFFFFu);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t x, uint64_t y) { return x > y ? x : y; }
template <int N>
__device__ __forceinline__ uint64_t ror_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)row_ror<N>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)row_ror<N>((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// M: experts per lane of a token's 16-lane row (E <= 16 M); NT threads.
template <int M, int NT>
__global__ __launch_bounds__(NT) void moe_route_kernel(MoeArgs a) {
    constexpr int kTok = NT / 16;          // tokens per pass
    constexpr int kMW = (kTok + 31) / 32;  // mask words per expert
    static_assert(kTok <= kRouteMaxTokens && kTok % 16 == 0, "tokens per pass");
    __shared__ int csel[kTok * kMaxTopK];    // this pass's picks
    __shared__ float cval[kTok * kMaxTopK];  // and their logits
    __shared__ uint32_t mask[kMaxExperts * kMW];     // bit (e, token of the pass)
    __shared__ int cnt[kMaxExperts];                 // pairs per expert so far (0 past E)
    __shared__ int loffs[kMaxExperts + 1];
    __shared__ int lpk[kRouteLdsPairs];              // packed pairs if they fit
    const int tid = threadIdx.x;
    const int sub = tid & 15;  // lane within the token's 16-lane row
    const int row = tid >> 4;  // token of the pass
    const int E = a.E, k = a.k, T = a.T, Pn = T * k;
    const int E4 = (E + 3) / 4 * 4;
    int* pk = Pn <= kRouteLdsPairs ? lpk : a.sel;  // rank << 9 | expert of pair (t, j)
    for (int e = tid; e < E4; e += NT) cnt[e] = 0;
    // this pass's logits (rows past T read row T - 1, experts past E read
    // expert E - 1; both are masked below), the next pass's issued before
    // this pass's picks
    float v[M];
    {
        const float* L = a.logits + (int64_t)min(row, T - 1) * E;
#pragma unroll
        for (int m = 0; m < M; ++m) v[m] = L[min(sub + 16 * m, E - 1)];
    }
    for (int t0 = 0; t0 < T; t0 += kTok) {
        const int t = t0 + row;
        const bool live = t < T;  // uniform over the 16-lane row
        uint64_t key[M];  // 0 past E: below every real key
#pragma unroll
        for (int m = 0; m < M; ++m) key[m] = sub + 16 * m < E ? route_key(v[m], sub + 16 * m) : 0ull;
        if (t0 + kTok < T) {
            const float* L = a.logits + (int64_t)min(t + kTok, T - 1) * E;
#pragma unroll
            for (int m = 0; m < M; ++m) v[m] = L[min(sub + 16 * m, E - 1)];
        }
        for (int w = tid; w < kMW * E; w += NT) mask[w] = 0;
        uint64_t prev = ~0ull;
        for (int j = 0; j < k; ++j) {
            // the largest key below the previous pick, over the lane, then
            // over the 16-lane row (rotations by 8, 4, 2, 1: every lane
            // ends with the row's maximum)
            uint64_t best = 0;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint64_t c = key[m] < prev ? key[m] : 0ull;
                best = c > best ? c : best;
            }
            best = max_u64(best, ror_u64<8>(best));
            best = max_u64(best, ror_u64<4>(best));
            best = max_u64(best, ror_u64<2>(best));
            best = max_u64(best, ror_u64<1>(best));
            prev = best;
            if (sub == 0) {
                csel[row * kMaxTopK + j] = key_expert(best);
                cval[row * kMaxTopK + j] = key_logit(best);
            }
        }
        if (live && sub == 0) {  // combine weights: softmax over the k picks
            const float* sv = cval + row * kMaxTopK;
            float sum = 0.0f;
            for (int j = 0; j < k; ++j) sum += expf(sv[j] - sv[0]);
            for (int j = 0; j < k; ++j) a.wgt[t * k + j] = expf(sv[j] - sv[0]) / sum;
        }
        __syncthreads();
        const int np = min(kTok, T - t0) * k;  // pairs of this pass
        for (int q = tid; q < np; q += NT) {
            const int r = q / k, e = csel[r * kMaxTopK + q % k];
            atomicOr(&mask[kMW * e + (r >> 5)], 1u << (r & 31));
        }
        __syncthreads();
        for (int q = tid; q < np; q += NT) {
            const int r = q / k, e = csel[r * kMaxTopK + q % k];
            const uint32_t* me = mask + kMW * e;
            int below = __popc(me[r >> 5] & ((1u << (r & 31)) - 1u));
            if (kMW == 2 && r >= 32) below += __popc(me[0]);
            pk[t0 * k + q] = ((cnt[e] + below) << 9) | e;
        }
        __syncthreads();
        for (int e = tid; e < E; e += NT) {
            int c = __popc(mask[kMW * e]);
            if (kMW == 2) c += __popc(mask[kMW * e + 1]);
            cnt[e] += c;
        }
        __syncthreads();
    }
    // offsets: one wave scans the counts (a lane sums a run of up to 8
    // experts, the lanes' totals are scanned across the wave)
    if (tid < 64) {
        const int run = (E + 63) / 64;
        const int e0 = tid * run, e1 = min(E, e0 + run);
        int tot = 0;
        for (int e = e0; e < e1; ++e) tot += cnt[e];
        int inc = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(inc, d, 64);
            if (tid >= d) inc += y;
        }
        int base = inc - tot;
        for (int e = e0; e < e1; ++e) {
            loffs[e] = base;
            base += cnt[e];
        }
        if (tid == 63) loffs[E] = inc;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += NT) a.offs[e] = loffs[e];
    for (int q = tid; q < Pn; q += NT) {
        const int pv = pk[q];
        const int pos = loffs[pv & 511] + (pv >> 9);
        a.prow[pos] = q / k;
        a.slot[q] = pos;
    }
}

// Stage 1 blocks (row block, expert, projection: z = 0 gate, 1 up); the
// tile's chunks of 8 groups and four blocks per CU as in the grouped launch.
constexpr int kLayerCG = 8;

template <int GB, int UB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
moe_gate_up_kernel(MoeArgs a) {
    constexpr int kW = (GB == 4 || UB == 4) ? Geo<4, kLayerCG>::kWRow : Geo<3, kLayerCG>::kWRow;
    __shared__ TileLds<kW, kLayerCG> lds;
    const int P = a.T * a.k;
    const int32_t G = (a.D + kGroup - 1) / kGroup;
    const bool up = blockIdx.z == 1;
    const uint8_t* pk = up ? a.up : a.gp;
    const float* sc = up ? a.us : a.gs;
    float* Y = up ? a.Yu : a.Yg;
    if constexpr (GB == UB) {
        grouped_tile<GB, true, true>(lds, blockIdx.y, blockIdx.x, pk, sc, a.F, a.D, G, a.X, a.T,
                                     a.prow, a.offs, P, Y);
    } else if (up) {
        grouped_tile<UB, true, true>(lds, blockIdx.y, blockIdx.x, pk, sc, a.F, a.D, G, a.X, a.T,
                                     a.prow, a.offs, P, Y);
    } else {
        grouped_tile<GB, true, true>(lds, blockIdx.y, blockIdx.x, pk, sc, a.F, a.D, G, a.X, a.T,
                                     a.prow, a.offs, P, Y);
    }
}

// Stage 2: h = silu(g) * u, four elements per thread (P * F % 4 == 0).
__global__ __launch_bounds__(256) void moe_swiglu_kernel(const float4* __restrict__ g,
                                                         const float4* __restrict__ u,
                                                         float4* __restrict__ h, int64_t n4) {
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4;
         q += (int64_t)gridDim.x * 256) {
        const float4 gv = g[q], uv = u[q];
        h[q] = make_float4(silu(gv.x) * uv.x, silu(gv.y) * uv.y, silu(gv.z) * uv.z,
                           silu(gv.w) * uv.w);
    }
}

// Stage 4: out[t][o] = sum_j w_tj * Yd[slot(t, j)][o], j in order; blocks
// (column block, tokens y, y + gridDim.y, ...), four columns per thread
// (D % 128 == 0).
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
    const int32_t o4 = blockIdx.x * 256 + threadIdx.x;
    if (4 * o4 >= a.D) return;
    for (int64_t t = blockIdx.y; t < a.T; t += gridDim.y) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < a.k; ++j) {
            const float w = a.wgt[t * a.k + j];
            const float4 y =
                reinterpret_cast<const float4*>(a.Yd + (int64_t)a.slot[t * a.k + j] * a.D)[o4];
            acc.x += w * y.x;
            acc.y += w * y.y;
            acc.z += w * y.z;
            acc.w += w * y.w;
        }
        reinterpret_cast<float4*>(a.out + t * a.D)[o4] = acc;
    }
}

}  // namespace

size_t moe_layer_workspace(int64_t T, int64_t k, int64_t E, int64_t D, int64_t F) {
    const int64_t P = T * k;
    auto up16 = [](int64_t b) { return (b + 15) / 16 * 16; };
    return (size_t)(4 * up16(P * 4) + up16((E + 1) * 4) + up16(3 * P * F * 4) +
                    up16(P * D * 4));
}

hipError_t launch_moe_layer(const float* X, int64_t T, int64_t D, int64_t F,
                            const float* logits, int32_t E, int32_t k, const uint8_t* gp,
                            const float* gs, int gbits, const uint8_t* up, const float* us,
                            int ubits, const uint8_t* dp, const float* ds, int dbits, float* out,
                            void* workspace, hipStream_t s) {
    if (k > kMaxTopK || E > kMaxExperts || T > (1 << 22)) return hipErrorInvalidValue;
    const int64_t P = T * k;
    auto up16 = [](int64_t b) { return (b + 15) / 16 * 16; };
    uint8_t* w = static_cast<uint8_t*>(workspace);
    MoeArgs a;
    a.X = X;
    a.logits = logits;
    a.T = (int32_t)T;
    a.D = (int32_t)D;
    a.F = (int32_t)F;
    a.E = E;
    a.k = k;
    a.gp = gp;
    a.gs = gs;
    a.up = up;
    a.us = us;
    a.dp = dp;
    a.ds = ds;
    a.gbits = gbits;
    a.ubits = ubits;
    a.dbits = dbits;
    a.out = out;
    a.sel = reinterpret_cast<int32_t*>(w);
    w += up16(P * 4);
    a.wgt = reinterpret_cast<float*>(w);
    w += up16(P * 4);
    a.slot = reinterpret_cast<int32_t*>(w);
    w += up16(P * 4);
    a.prow = reinterpret_cast<int32_t*>(w);
    w += up16(P * 4);
    a.offs = reinterpret_cast<int32_t*>(w);
    w += up16((E + 1) * 4);
    a.Yg = reinterpret_cast<float*>(w);
    a.Yu = a.Yg + P * F;
    a.H = a.Yu + P * F;
    w += up16(3 * P * F * 4);
    a.Yd = reinterpret_cast<float*>(w);

    if (gbits < 3 || gbits > 4 || ubits < 3 || ubits > 4 || dbits < 3 || dbits > 4)
        return hipErrorInvalidValue;
    if (E <= 128)
        moe_route_kernel<8, 1024><<<1, 1024, 0, s>>>(a);
    else if (E <= 256)
        moe_route_kernel<16, 512><<<1, 512, 0, s>>>(a);
    else
        moe_route_kernel<32, 256><<<1, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    const dim3 grid1((unsigned)((F + kRows - 1) / kRows), (unsigned)E, 2);
    if (gbits == 3 && ubits == 3)
        moe_gate_up_kernel<3, 3><<<grid1, kThreads, 0, s>>>(a);
    else if (gbits == 3)
        moe_gate_up_kernel<3, 4><<<grid1, kThreads, 0, s>>>(a);
    else if (ubits == 3)
        moe_gate_up_kernel<4, 3><<<grid1, kThreads, 0, s>>>(a);
    else
        moe_gate_up_kernel<4, 4><<<grid1, kThreads, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const int64_t n4 = P * F / 4;  // F % 128 == 0
    moe_swiglu_kernel<<<(unsigned)std::min<int64_t>((n4 + 255) / 256, 4096), 256, 0, s>>>(
        reinterpret_cast<const float4*>(a.Yg), reinterpret_cast<const float4*>(a.Yu),
        reinterpret_cast<float4*>(a.H), n4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    e = launch_gemv_grouped(dp, ds, E, D, F, a.H, P, nullptr, a.offs, (int32_t)P, a.Yd, s, dbits);
    if (e != hipSuccess) return e;

    const dim3 grid4((unsigned)((D / 4 + 255) / 256), (unsigned)std::min<int64_t>(T, 65535));
    moe_combine_kernel<<<grid4, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace qt
