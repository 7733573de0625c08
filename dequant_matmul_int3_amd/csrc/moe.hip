// A mixture-of-experts expert layer in two launches: a one-block routing
// kernel, then a persistent kernel for the gate and up projections, SwiGLU,
// the down projection and the combine of every token's experts (the pull
// request page's MoE decode setting: every routed expert's weights read once
// per step; its per-projection ablation names gate_proj, up_proj and
// down_proj, each at int3-g64 or grouped int4).
//
//  0. routing (its own launch, one block): per token the k largest logits
//     (equal logits: lower expert first), combine weights a softmax over
//     them; the (expert, token) pairs sorted by expert, then token; the
//     expert work order; the phase counters of the layer kernel zeroed.
// Then phases separated by grid-wide barriers (a cooperative launch, so
// every block of the grid is resident; no block leaves before the last
// barrier):
//  1. items (expert, 64-row block of gate and up): the grouped matrix-core
//     tile for gate, then for up, then h = silu(g) * u for those rows of
//     every pair of the expert.
//  2. items (expert, 64-row block of down): the same tile on h.
//  3. out[t] = sum_j w_tj y_{pair(t, j)} in j order.
// A block's first item of a phase is its block index; later ones come from
// the phase's shared counter as blocks finish, in the routing's expert order
// (the most pairs first, so the longest items start early); experts without
// pairs have no items.  Each item writes its own outputs, so the results do
// not depend on which block ran it.  (Routing inside the persistent kernel
// cost a grid barrier that every block reached at once, which measured
// tens of microseconds.)
#include <hip/hip_cooperative_groups.h>

#include "grouped_tile.h"

namespace qt {
namespace {

namespace cg = cooperative_groups;

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
    int32_t* order;  // [E] experts with pairs, most pairs first (ties: lower index)
    int32_t* ctr;    // [4] next gate/up item, next down item, experts with pairs
    float* Yg;       // [P x F]
    float* Yu;       // [P x F]
    float* H;        // [P x F] silu(g) * u
    float* Yd;       // [P x D]
};

// Phase 0, one block of NT threads: 16 lanes per token, NT / 16 tokens per
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
    __shared__ int s_ne;
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
        if (tid == 0) s_ne = 0;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += NT) a.offs[e] = loffs[e];
    for (int q = tid; q < Pn; q += NT) {
        const int pv = pk[q];
        const int pos = loffs[pv & 511] + (pv >> 9);
        a.prow[pos] = q / k;
        a.slot[q] = pos;
    }
    // the work order of the expert phases: experts with pairs, the most
    // first (their items take longest), ties by index
    for (int e = tid; e < E; e += NT) {
        const int c = cnt[e];
        if (c > 0) {
            int rank = 0;
            for (int e2 = 0; e2 < E4; e2 += 4) {  // four counts per LDS read
                const int4 c4 = *reinterpret_cast<const int4*>(cnt + e2);
                rank += (c4.x > c) || (c4.x == c && e2 < e);
                rank += (c4.y > c) || (c4.y == c && e2 + 1 < e);
                rank += (c4.z > c) || (c4.z == c && e2 + 2 < e);
                rank += (c4.w > c) || (c4.w == c && e2 + 3 < e);
            }
            a.order[rank] = e;
            atomicAdd(&s_ne, 1);
        }
    }
    __syncthreads();
    if (tid == 0) {  // the layer kernel's phase counters
        a.ctr[0] = 0;
        a.ctr[1] = 0;
        a.ctr[2] = s_ne;
    }
}

// Work items of a phase come from the phase's shared counter as blocks
// finish (uneven items leave no long tail).  The counter is read one step
// ahead: ask() issues the atomic in thread 0 and keeps the result in a
// register, take() hands it to the block, so the atomic's latency overlaps
// the work issued in between.
struct ItemCounter {
    int32_t* ctr;
    int32_t pending;  // thread 0 only
    __device__ __forceinline__ void ask() {
        if (threadIdx.x == 0) pending = atomicAdd(ctr, 1);
    }
    __device__ __forceinline__ int64_t take() {
        __shared__ int32_t s_item;
        if (threadIdx.x == 0) s_item = pending;
        __syncthreads();
        const int64_t it = s_item;
        __syncthreads();  // everyone has read it before the next take()
        return it;
    }
};

// Sixteen groups per chunk: the layer's kernel holds two blocks per CU either
// way (its registers), so fewer chunk barriers win (eight-group chunks for
// the down tiles, a second tile instantiation in the kernel, raised its
// registers to one block per CU for some formats).
constexpr int kLayerCG = 16;

template <int BITS, int WROW, int CG>
__device__ __forceinline__ void tile_bits(TileLds<WROW, CG>& L, int e, int64_t rb,
                                          const uint8_t* packed, const float* scales, int64_t O,
                                          int32_t I, const float* X, int64_t nx,
                                          const int32_t* prow, const int32_t* offs, int32_t P,
                                          float* Y) {
    const int32_t G = (I + kGroup - 1) / kGroup;
    grouped_tile<BITS, true, true, WROW, CG, false>(L, e, rb, packed, scales, O, I, G, X, nx, prow,
                                                   offs, P, Y);
}

// Routing tables the items look up, copied to LDS at the start (a global
// read each time put its latency on every item's critical path): the expert
// order, the offsets and, up to this many pairs, the pairs' token rows.
constexpr int kLayerLdsPairs = 1024;

// GB, UB, DB: the formats (3 or 4 bits) of gate, up and down.
template <int GB, int UB, int DB>
__global__ __launch_bounds__(kThreads, 2) void moe_layer_kernel(MoeArgs a) {
    constexpr int kW = (GB == 4 || UB == 4 || DB == 4) ? Geo<4, kLayerCG>::kWRow
                                                       : Geo<3, kLayerCG>::kWRow;
    __shared__ TileLds<kW, kLayerCG> lds;
    __shared__ int32_t s_order[kMaxExperts];
    __shared__ int32_t s_offs[kMaxExperts + 1];
    __shared__ int32_t s_prow[kLayerLdsPairs];
    cg::grid_group grid = cg::this_grid();
    const int P = a.T * a.k;
    const int tid = threadIdx.x;

    const int64_t nf = (a.F + kRows - 1) / kRows, nd = (a.D + kRows - 1) / kRows;
    const int64_t ne = a.ctr[2];
    ItemCounter c1{&a.ctr[0], 0};
    for (int i = tid; i < ne; i += kThreads) s_order[i] = a.order[i];
    for (int i = tid; i <= a.E; i += kThreads) s_offs[i] = a.offs[i];
    const bool prow_lds = P <= kLayerLdsPairs;
    if (prow_lds)
        for (int i = tid; i < P; i += kThreads) s_prow[i] = a.prow[i];
    const int32_t* prow = prow_lds ? s_prow : a.prow;
    __syncthreads();

    const int64_t items1 = ne * nf;
    for (int64_t it = blockIdx.x; it < items1;) {
        const int e = s_order[it / nf];
        const int64_t rb = it % nf;
        tile_bits<GB>(lds, e, rb, a.gp, a.gs, a.F, a.D, a.X, a.T, prow, s_offs, P, a.Yg);
        tile_bits<UB>(lds, e, rb, a.up, a.us, a.F, a.D, a.X, a.T, prow, s_offs, P, a.Yu);
        // h for this block's rows of every pair of the expert (the tiles'
        // stores above come from this block: a barrier makes them visible);
        // the next item is asked for first (items here are long: asking
        // earlier could leave a block holding one while others idle); every
        // answer is taken below, so no item is skipped
        c1.ask();
        const int p0 = s_offs[e], p1 = s_offs[e + 1];
        __syncthreads();
        const int64_t r0 = rb * kRows;
        for (int q = tid; q < (p1 - p0) * kRows; q += kThreads) {
            const int64_t p = p0 + q / kRows, r = r0 + q % kRows;
            if (r < a.F) a.H[p * a.F + r] = silu(a.Yg[p * a.F + r]) * a.Yu[p * a.F + r];
        }
        it = gridDim.x + c1.take();
    }
    grid.sync();

    const int64_t items2 = ne * nd;
    ItemCounter c2{&a.ctr[1], 0};
    for (int64_t it = blockIdx.x; it < items2;) {
        c2.ask();  // short items: the next one is asked for as this one starts (taken below)
        const int e = s_order[it / nd];
        const int64_t rb = it % nd;
        tile_bits<DB>(lds, e, rb, a.dp, a.ds, a.D, a.F, a.H, P, nullptr, s_offs, P, a.Yd);
        it = gridDim.x + c2.take();
    }
    grid.sync();

    const int64_t n = (int64_t)a.T * a.D;
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < n;
         q += (int64_t)gridDim.x * kThreads) {
        const int64_t t = q / a.D, o = q % a.D;
        float acc = 0.0f;
        for (int j = 0; j < a.k; ++j)
            acc += a.wgt[t * a.k + j] * a.Yd[(int64_t)a.slot[t * a.k + j] * a.D + o];
        a.out[q] = acc;
    }
}

}  // namespace

size_t moe_layer_workspace(int64_t T, int64_t k, int64_t E, int64_t D, int64_t F) {
    const int64_t P = T * k;
    auto up16 = [](int64_t b) { return (b + 15) / 16 * 16; };
    return (size_t)(4 * up16(P * 4) + up16((E + 1) * 4) + up16(E * 4) + up16(4 * 4) +
                    up16(3 * P * F * 4) + up16(P * D * 4));
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
    a.order = reinterpret_cast<int32_t*>(w);
    w += up16(E * 4);
    a.ctr = reinterpret_cast<int32_t*>(w);
    w += up16(4 * 4);
    a.Yg = reinterpret_cast<float*>(w);
    a.Yu = a.Yg + P * F;
    a.H = a.Yu + P * F;
    w += up16(3 * P * F * 4);
    a.Yd = reinterpret_cast<float*>(w);

    const int code = (gbits - 3) * 4 + (ubits - 3) * 2 + (dbits - 3);
    const void* kernels[8] = {
        reinterpret_cast<const void*>(moe_layer_kernel<3, 3, 3>),
        reinterpret_cast<const void*>(moe_layer_kernel<3, 3, 4>),
        reinterpret_cast<const void*>(moe_layer_kernel<3, 4, 3>),
        reinterpret_cast<const void*>(moe_layer_kernel<3, 4, 4>),
        reinterpret_cast<const void*>(moe_layer_kernel<4, 3, 3>),
        reinterpret_cast<const void*>(moe_layer_kernel<4, 3, 4>),
        reinterpret_cast<const void*>(moe_layer_kernel<4, 4, 3>),
        reinterpret_cast<const void*>(moe_layer_kernel<4, 4, 4>)};
    if (code < 0 || code > 7) return hipErrorInvalidValue;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernels[code], kThreads, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
    if (E <= 128)
        moe_route_kernel<8, 1024><<<1, 1024, 0, s>>>(a);
    else if (E <= 256)
        moe_route_kernel<16, 512><<<1, 512, 0, s>>>(a);
    else
        moe_route_kernel<32, 256><<<1, 256, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    return hipLaunchCooperativeKernel(kernels[code], dim3((unsigned)(per_cu * cus)), dim3(kThreads),
                                      args, 0, s);
}

}  // namespace qt
