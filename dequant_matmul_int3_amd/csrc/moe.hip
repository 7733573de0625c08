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
//     token) pairs sorted by expert, then token.
//  1. items (gate | up, expert, 64-row block): the grouped matrix-core tile,
//     g and u for every pair of the expert.
//  2. items (expert, 64-row block of down): the same tile on the inputs
//     h = silu(g) * u, formed as they are loaded (no h buffer, no pass).
//  3. out[t] = sum_j w_tj y_{pair(t, j)} in j order.
// Items are dealt round-robin over the blocks; experts without pairs cost a
// read of two offsets.
#include <hip/hip_cooperative_groups.h>

#include "grouped_tile.h"

namespace qt {
namespace {

namespace cg = cooperative_groups;

constexpr int kMaxTopK = 32;

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
    float* Yd;       // [P x D]
};

// Phase 0, one block.
__device__ void route(const MoeArgs& a) {
    const int tid = threadIdx.x;
    const int E = a.E, k = a.k;
    for (int t = tid; t < a.T; t += kThreads) {
        const float* L = a.logits + (int64_t)t * E;
        float sv[kMaxTopK];
        int si[kMaxTopK];
        // the j-th pick: the smallest key (-logit, expert) above the previous
        float pv = 0.0f;
        int pi = -1;
        for (int j = 0; j < k; ++j) {
            float bv = 0.0f;
            int bi = -1;
            for (int e = 0; e < E; ++e) {
                const float v = L[e];
                const bool after = pi < 0 || v < pv || (v == pv && e > pi);
                if (after && (bi < 0 || v > bv)) {  // ascending e: ties keep the lower
                    bv = v;
                    bi = e;
                }
            }
            sv[j] = bv;
            si[j] = bi;
            pv = bv;
            pi = bi;
        }
        float z[kMaxTopK];
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) {
            z[j] = expf(sv[j] - sv[0]);
            sum += z[j];
        }
        for (int j = 0; j < k; ++j) {
            a.sel[t * k + j] = si[j];
            a.wgt[t * k + j] = z[j] / sum;
        }
    }
    __syncthreads();
    // counts per expert, then offsets (one thread), then placement in token order
    for (int e = tid; e < E; e += kThreads) {
        int c = 0;
        for (int q = 0; q < a.T * k; ++q) c += a.sel[q] == e;
        a.offs[e + 1] = c;
    }
    __syncthreads();
    if (tid == 0) {
        a.offs[0] = 0;
        for (int e = 0; e < E; ++e) a.offs[e + 1] += a.offs[e];
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
        int pos = a.offs[e];
        for (int q = 0; q < a.T * k; ++q)
            if (a.sel[q] == e) {
                a.prow[pos] = q / k;
                a.slot[q] = pos;
                ++pos;
            }
    }
}

template <int XF>
__device__ __forceinline__ void tile_bits(TileLds<Geo<4>::kWRow>& L, int bits, int e, int64_t rb,
                                          const uint8_t* packed, const float* scales, int64_t O,
                                          int32_t I, const float* X, const float* X2,
                                          int64_t nx, const int32_t* prow, const int32_t* offs,
                                          int32_t P, float* Y) {
    const int32_t G = (I + kGroup - 1) / kGroup;
    if (bits == 3)
        grouped_tile<3, true, true, XF>(L, e, rb, packed, scales, O, I, G, X, X2, nx, prow, offs,
                                        P, Y);
    else
        grouped_tile<4, true, true, XF>(L, e, rb, packed, scales, O, I, G, X, X2, nx, prow, offs,
                                        P, Y);
}

__global__ __launch_bounds__(kThreads) void moe_layer_kernel(MoeArgs a) {
    __shared__ TileLds<Geo<4>::kWRow> lds;
    cg::grid_group grid = cg::this_grid();
    const int P = a.T * a.k;
    if (blockIdx.x == 0) route(a);
    grid.sync();

    const int64_t nf = (a.F + kRows - 1) / kRows, nd = (a.D + kRows - 1) / kRows;
    const int64_t items1 = 2 * a.E * nf;
    for (int64_t it = blockIdx.x; it < items1; it += gridDim.x) {
        const int proj = (int)(it / (a.E * nf));
        const int64_t rem = it % (a.E * nf);
        const int e = (int)(rem / nf);
        const int64_t rb = rem % nf;
        if (proj == 0)
            tile_bits<kPlain>(lds, a.gbits, e, rb, a.gp, a.gs, a.F, a.D, a.X, nullptr, a.T, a.prow,
                              a.offs, P, a.Yg);
        else
            tile_bits<kPlain>(lds, a.ubits, e, rb, a.up, a.us, a.F, a.D, a.X, nullptr, a.T, a.prow,
                              a.offs, P, a.Yu);
    }
    grid.sync();

    const int64_t items2 = a.E * nd;
    for (int64_t it = blockIdx.x; it < items2; it += gridDim.x) {
        const int e = (int)(it / nd);
        const int64_t rb = it % nd;
        tile_bits<kSwiGLU>(lds, a.dbits, e, rb, a.dp, a.ds, a.D, a.F, a.Yg, a.Yu, P, nullptr,
                           a.offs, P, a.Yd);
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
    return (size_t)(4 * up16(P * 4) + up16((E + 1) * 4) + up16(2 * P * F * 4) + up16(P * D * 4));
}

hipError_t launch_moe_layer(const float* X, int64_t T, int64_t D, int64_t F,
                            const float* logits, int32_t E, int32_t k, const uint8_t* gp,
                            const float* gs, int gbits, const uint8_t* up, const float* us,
                            int ubits, const uint8_t* dp, const float* ds, int dbits, float* out,
                            void* workspace, hipStream_t s) {
    if (k > kMaxTopK) return hipErrorInvalidValue;
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
    w += up16(2 * P * F * 4);
    a.Yd = reinterpret_cast<float*>(w);

    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_layer_kernel, kThreads, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
    void* args[] = {&a};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(moe_layer_kernel),
                                      dim3((unsigned)(per_cu * cus)), dim3(kThreads), args, 0, s);
}

}  // namespace qt
