// A mixture-of-experts expert layer in one persistent launch: routing, the
// gate and up projections, SwiGLU, the down projection and the combine of
// every token's experts (the pull request page's MoE decode setting: every
// routed expert's weights read once per step; its per-projection ablation
// names gate_proj, up_proj and down_proj, each at int3-g64 or grouped int4).
//
// Phases, separated by grid-wide barriers (a cooperative launch, so every
// block of the grid is resident; no block leaves before the last barrier):
//  0. block 0 routes: per token the k largest logits (equal logits: lower
//     expert first), combine weights a softmax over them; the (expert,
//     token) pairs sorted by expert, then token; the expert work order.
//  1. items (expert, 64-row block of gate and up): the grouped matrix-core
//     tile for gate, then for up, then h = silu(g) * u for those rows of
//     every pair of the expert.
//  2. items (expert, 64-row block of down): the same tile on h.
//  3. out[t] = sum_j w_tj y_{pair(t, j)} in j order.
// Blocks take the items of a phase from a shared counter as they finish, in
// the routing's expert order (the most pairs first, so the longest items
// start early); experts without pairs have no items.  Each item writes its
// own outputs, so the results do not depend on which block ran it.
#include <hip/hip_cooperative_groups.h>

#include "grouped_tile.h"

namespace qt {
namespace {

namespace cg = cooperative_groups;

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 512;  // routing keeps a token's logits in registers (32 per lane)
constexpr int kRouteLdsPairs = (20 * 1024 - 16 * 32 * 4 - 2 * 256 * 4) / 4;  // selections in LDS

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

// Phase 0, one block: a wave per token picks its k experts one at a time
// (each pick the largest logit after the previous one in the order
// (-logit, expert): the lanes scan the logits, a butterfly keeps the larger,
// on equal logits the lower expert); then counts per expert (order-free
// atomics), offsets, and each pair's slot = its expert's offset + the number
// of earlier tokens that chose the same expert.
// value of lane (l - N) mod 16 of this lane's 16-lane row
template <int N>
__device__ __forceinline__ int row_ror(int v) {
    return __builtin_amdgcn_mov_dpp(v, 0x120 + N, 0xF, 0xF, false);
}

__device__ void route(const MoeArgs& a, uint8_t* scratch /* >= 20 KB of LDS */) {
    const int tid = threadIdx.x;
    const int sub = tid & 15;              // lane within the token's 16-lane row
    const int row = tid >> 4;              // 16 tokens in flight per block
    const int E = a.E, k = a.k, Pn = a.T * a.k;
    float* svals = reinterpret_cast<float*>(scratch);           // [16][kMaxTopK]
    int* part = reinterpret_cast<int*>(scratch + 16 * kMaxTopK * 4);  // [2][kThreads] scan
    int* lsel = part + 2 * kThreads;                             // [Pn] if it fits
    const bool sel_in_lds = Pn <= kRouteLdsPairs;
    for (int e = tid; e <= E; e += kThreads) a.offs[e] = 0;
    for (int t0 = 0; t0 < a.T; t0 += kThreads / 16) {
        const int t = t0 + row;
        const bool live = t < a.T;  // uniform over the 16-lane row
        const float* L = a.logits + (int64_t)(live ? t : 0) * E;
        float lv[kMaxExperts / 16];  // logits sub + 16 m, read once
#pragma unroll
        for (int m = 0; m < kMaxExperts / 16; ++m) {
            const int e = sub + 16 * m;
            lv[m] = e < E ? L[e] : 0.0f;
        }
        float pv = 0.0f;
        int pi = -1;
        for (int j = 0; j < k; ++j) {
            float bv = 0.0f;
            int bi = -1;
#pragma unroll
            for (int m = 0; m < kMaxExperts / 16; ++m) {
                const int e = sub + 16 * m;
                const float v = lv[m];
                const bool after = pi < 0 || v < pv || (v == pv && e > pi);
                if (e < E && after && (bi < 0 || v > bv)) {  // ascending e: ties keep the lower
                    bv = v;
                    bi = e;
                }
            }
            // all 16 lanes of the row end with the row's best (rotations by
            // 8, 4, 2, 1 combine every lane's candidate)
#define QT_ROUTE_STEP(N)                                                              \
    {                                                                                 \
        const float ov = __int_as_float(row_ror<N>(__float_as_int(bv)));              \
        const int oi = row_ror<N>(bi);                                                \
        if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {                 \
            bv = ov;                                                                  \
            bi = oi;                                                                  \
        }                                                                             \
    }
            QT_ROUTE_STEP(8)
            QT_ROUTE_STEP(4)
            QT_ROUTE_STEP(2)
            QT_ROUTE_STEP(1)
#undef QT_ROUTE_STEP
            pv = bv;
            pi = bi;
            if (live && sub == 0) {
                a.sel[t * k + j] = bi;
                if (sel_in_lds) lsel[t * k + j] = bi;
                svals[row * kMaxTopK + j] = bv;
            }
        }
        if (live && sub == 0) {  // combine weights: softmax over the k picks
            const float* sv = svals + row * kMaxTopK;
            float sum = 0.0f;
            for (int j = 0; j < k; ++j) sum += expf(sv[j] - sv[0]);
            for (int j = 0; j < k; ++j) a.wgt[t * k + j] = expf(sv[j] - sv[0]) / sum;
        }
    }
    __syncthreads();
    const int* sel = sel_in_lds ? lsel : a.sel;
    for (int q = tid; q < Pn; q += kThreads) atomicAdd(&a.offs[sel[q] + 1], 1);
    __syncthreads();
    // offsets: each thread totals a contiguous run of experts, the totals
    // are scanned in LDS (log steps), then each run is rewritten from its base
    const int run = (E + kThreads - 1) / kThreads;
    const int e0 = tid * run, e1 = min(E, e0 + run);
    int tot = 0;
    for (int e = e0; e < e1; ++e) tot += a.offs[e + 1];
    part[tid] = tot;
    __syncthreads();
    int cur = 0;
    for (int d = 1; d < kThreads; d <<= 1) {
        const int v = part[cur * kThreads + tid] + (tid >= d ? part[cur * kThreads + tid - d] : 0);
        part[(cur ^ 1) * kThreads + tid] = v;
        cur ^= 1;
        __syncthreads();
    }
    int base = tid > 0 ? part[cur * kThreads + tid - 1] : 0;
    for (int e = e0; e < e1; ++e) {
        base += a.offs[e + 1];
        a.offs[e + 1] = base;
    }
    __syncthreads();
    for (int q = tid; q < Pn; q += kThreads) {
        const int e = sel[q], t = q / k;
        int rank = 0;
        for (int q2 = 0; q2 < t * k; ++q2) rank += sel[q2] == e;  // a token picks e at most once
        const int pos = a.offs[e] + rank;
        a.prow[pos] = t;
        a.slot[q] = pos;
    }
    // the work order of the expert phases: experts with pairs, the most
    // first (their items take longest), ties by index; the work counters
    // start at zero
    int* cnt = part;  // [E] pair counts (the scan is done with part)
    for (int e = tid; e < E; e += kThreads) cnt[e] = a.offs[e + 1] - a.offs[e];
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
        const int c = cnt[e];
        if (c > 0) {
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2) {
                const int c2 = cnt[e2];
                rank += (c2 > c) || (c2 == c && e2 < e);
            }
            a.order[rank] = e;
        }
    }
    if (tid == 0) {
        int ne = 0;
        for (int e = 0; e < E; ++e) ne += cnt[e] > 0;
        a.ctr[0] = 0;
        a.ctr[1] = 0;
        a.ctr[2] = ne;
    }
}

// The next item of a phase for this block, from the phase's shared counter
// (blocks take items as they finish, so uneven items leave no long tail).
__device__ __forceinline__ int64_t next_item(int32_t* ctr) {
    __shared__ int32_t s_item;
    if (threadIdx.x == 0) s_item = atomicAdd(ctr, 1);
    __syncthreads();
    const int64_t it = s_item;
    __syncthreads();  // everyone has read it before the next call overwrites it
    return it;
}

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
    grouped_tile<BITS, true, true>(L, e, rb, packed, scales, O, I, G, X, nx, prow, offs, P, Y);
}

// GB, UB, DB: the formats (3 or 4 bits) of gate, up and down.
template <int GB, int UB, int DB>
__global__ __launch_bounds__(kThreads) void moe_layer_kernel(MoeArgs a) {
    constexpr int kW = (GB == 4 || UB == 4 || DB == 4) ? Geo<4, kLayerCG>::kWRow
                                                       : Geo<3, kLayerCG>::kWRow;
    __shared__ TileLds<kW, kLayerCG> lds;
    static_assert(sizeof(lds.wl) >= 20 * 1024, "the routing borrows 20 KB of the weight LDS");
    cg::grid_group grid = cg::this_grid();
    const int P = a.T * a.k;
    // the routing borrows the tile's weight LDS (no tile has run yet)
    if (blockIdx.x == 0) route(a, lds.wl);
    grid.sync();

    const int64_t nf = (a.F + kRows - 1) / kRows, nd = (a.D + kRows - 1) / kRows;
    const int64_t ne = a.ctr[2];
    const int64_t items1 = ne * nf;
    for (;;) {
        const int64_t it = next_item(&a.ctr[0]);
        if (it >= items1) break;  // uniform
        const int e = a.order[it / nf];
        const int64_t rb = it % nf;
        tile_bits<GB>(lds, e, rb, a.gp, a.gs, a.F, a.D, a.X, a.T, a.prow, a.offs, P, a.Yg);
        tile_bits<UB>(lds, e, rb, a.up, a.us, a.F, a.D, a.X, a.T, a.prow, a.offs, P, a.Yu);
        // h for this block's rows of every pair of the expert (the tiles'
        // stores above come from this block: a barrier makes them visible)
        const int p0 = a.offs[e], p1 = a.offs[e + 1];
        __syncthreads();
        const int64_t r0 = rb * kRows;
        for (int q = threadIdx.x; q < (p1 - p0) * kRows; q += kThreads) {
            const int64_t p = p0 + q / kRows, r = r0 + q % kRows;
            if (r < a.F) a.H[p * a.F + r] = silu(a.Yg[p * a.F + r]) * a.Yu[p * a.F + r];
        }
    }
    grid.sync();

    const int64_t items2 = ne * nd;
    for (;;) {
        const int64_t it = next_item(&a.ctr[1]);
        if (it >= items2) break;  // uniform
        const int e = a.order[it / nd];
        const int64_t rb = it % nd;
        tile_bits<DB>(lds, e, rb, a.dp, a.ds, a.D, a.F, a.H, P, nullptr, a.offs, P, a.Yd);
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
    if (k > kMaxTopK || E > kMaxExperts) return hipErrorInvalidValue;
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
    void* args[] = {&a};
    return hipLaunchCooperativeKernel(kernels[code], dim3((unsigned)(per_cu * cus)), dim3(kThreads),
                                      args, 0, s);
}

}  // namespace qt
