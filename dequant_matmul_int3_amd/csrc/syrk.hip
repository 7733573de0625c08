// The full Hessian H = sum_t X[t]^T X[t] of one linear input on the gfx950
// matrix cores (the tt-stack issue page, pipeline table step 1: rank-k
// accumulations over the calibration tokens, fp32 accumulation on the device).
//
// X [T x I] is first transposed into Xt [Ip x Tp] (rows padded to a multiple
// of 256 columns of X, tokens to a multiple of 64, padding zero), so that both
// MFMA operands read token-contiguous rows: H[i][j] = sum_t Xt[i][t] Xt[j][t].
// bf16 inputs go to v_mfma_f32_16x16x32_bf16 (every product exact, sums in
// f32); f32 inputs to v_mfma_f32_16x16x4_f32.  Only tiles on or above the
// diagonal are computed; each writes its values to both triangles, and a
// diagonal tile writes each pair once from its upper element, so H is
// exactly symmetric.
//
// bf16 inputs take a kernel of their own with 256 x 256 output tiles: 8 waves
// of 128 x 64.  Both operands go through LDS in MFMA operand order, in
// 32-token stages: each stage is loaded into registers two steps ahead and
// stored into its LDS slot one step ahead, with one barrier per step.  Only the tiles on or
// above the diagonal are launched, in strips of 8 tile rows walked column
// by column, and each XCD takes one contiguous run of that order, so the
// blocks resident on an XCD share their row blocks of Xt in its L2.
//
// The 128 x 128 NT kernel serves the f32 inputs and the GPTQ proxy terms:
// with A = [W; E] and B = H (symmetric, so its rows are its columns), each
// output tile reduces sum_n (A H)[m][n] A[m][n] per row into a partial, in a
// fixed order.
#include <algorithm>

#include "lds_barrier.h"
#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kTile = 128;    // output tile (rows and columns of H)
constexpr int kThreads = 256;  // 4 waves, 2 x 2 over the tile, 64 x 64 each
constexpr int kPadRows = 256;  // Xt rows padded to a multiple of this
constexpr int kPadK = 64;      // Xt columns (tokens) padded to a multiple of this

// 64 x 64 tile transpose through LDS: Xt[i][t] = X[t][i], zero outside X.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ X, int64_t Tn,
                                                         int64_t I, int64_t Tp,
                                                         T* __restrict__ Xt) {
    __shared__ T tile[64][65];
    const int64_t t0 = (int64_t)blockIdx.x * 64, i0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    for (int r = ty; r < 64; r += 4) {
        const int64_t t = t0 + r, i = i0 + tx;
        tile[r][tx] = (t < Tn && i < I) ? X[t * I + i] : T(0);
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t i = i0 + r, t = t0 + tx;
        Xt[i * Tp + t] = tile[tx][r];  // rows i < Ip, t < Tp: inside the padded buffer
    }
}

// Per K step of the LDS tile: bf16 64 tokens (two MFMA k-halves of 32), f32
// 16 tokens (four MFMA steps of 4).
template <bool BF16>
struct SyrkCfg {
    static constexpr int kK = BF16 ? 64 : 16;            // tokens per LDS stage
    static constexpr int kEsz = BF16 ? 2 : 4;
    static constexpr int kRowBytes = kK * kEsz;           // 128 or 64
    static constexpr int kPitch = kRowBytes + 16;         // LDS bytes per tile row
    static constexpr int kLoads = kTile * kRowBytes / 16 / kThreads;  // 16-byte loads per operand
};

enum NtMode { kSymStore, kRowDot };

// C = A B^T over row tiles of A (i0) and B (j0), both [rows x Kp] with row
// pitch Kp elements, rows padded to whole tiles and Kp to whole K stages.
// kSymStore: A = B = Xt, tiles with bi <= bj, C into H [I x I] (both
// triangles).  kRowDot: part[m][bj] = sum over the tile's columns n of
// C[m][n] * A[m][n] (A's column n is the K index n).
template <bool BF16, int MODE>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(const void* __restrict__ A_,
                                                           const void* __restrict__ B_,
                                                           int64_t Kp, int64_t I,
                                                           float* __restrict__ H,
                                                           int accumulate,
                                                           float* __restrict__ part) {
    using Cfg = SyrkCfg<BF16>;
    const int bi = blockIdx.y, bj = blockIdx.x;
    if (MODE == kSymStore && bi > bj) return;  // upper tiles only; uniform over the block
    __shared__ __attribute__((aligned(16))) uint8_t As[kTile * Cfg::kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[kTile * Cfg::kPitch];

    const uint8_t* Ab = static_cast<const uint8_t*>(A_);
    const uint8_t* Bb = static_cast<const uint8_t*>(B_);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t i0 = (int64_t)bi * kTile, j0 = (int64_t)bj * kTile;
    const int64_t rowb = Kp * Cfg::kEsz;  // bytes per row

    // staging: load l of this thread = 16-byte piece (tid + 256 l) of the
    // [128 rows][kRowBytes] tile
    int srow[Cfg::kLoads], scol[Cfg::kLoads];
#pragma unroll
    for (int l = 0; l < Cfg::kLoads; ++l) {
        const int id = tid + kThreads * l;
        srow[l] = id / (Cfg::kRowBytes / 16);
        scol[l] = (id % (Cfg::kRowBytes / 16)) * 16;
    }
    u32x4_t ra[Cfg::kLoads], rb[Cfg::kLoads];
    auto load = [&](int64_t k0) {  // k0 in tokens
#pragma unroll
        for (int l = 0; l < Cfg::kLoads; ++l) {
            const int64_t off = k0 * Cfg::kEsz + scol[l];
            ra[l] = *reinterpret_cast<const u32x4_t*>(Ab + (i0 + srow[l]) * rowb + off);
            rb[l] = *reinterpret_cast<const u32x4_t*>(Bb + (j0 + srow[l]) * rowb + off);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int l = 0; l < Cfg::kLoads; ++l) {
            *reinterpret_cast<u32x4_t*>(As + srow[l] * Cfg::kPitch + scol[l]) = ra[l];
            *reinterpret_cast<u32x4_t*>(Bs + srow[l] * Cfg::kPitch + scol[l]) = rb[l];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int l16 = lane & 15, lq = lane >> 4;
    load(0);
    for (int64_t k0 = 0; k0 < Kp; k0 += Cfg::kK) {
        __syncthreads();  // the previous stage is consumed
        store();
        __syncthreads();
        if (k0 + Cfg::kK < Kp) load(k0 + Cfg::kK);  // next stage in flight
        if constexpr (BF16) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4_t a[4], b[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int r = 64 * wm + 16 * m + l16;
                    a[m] = *reinterpret_cast<const u32x4_t*>(As + r * Cfg::kPitch + 64 * ks + 16 * lq);
                }
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const int r = 64 * wn + 16 * n + l16;
                    b[n] = *reinterpret_cast<const u32x4_t*>(Bs + r * Cfg::kPitch + 64 * ks + 16 * lq);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int n = 0; n < 4; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, a[m]), __builtin_bit_cast(bf16x8_t, b[n]),
                            acc[m][n], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float a[4], b[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int r = 64 * wm + 16 * m + l16;
                    a[m] = *reinterpret_cast<const float*>(As + r * Cfg::kPitch + 4 * (4 * ks + lq));
                }
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const int r = 64 * wn + 16 * n + l16;
                    b[n] = *reinterpret_cast<const float*>(Bs + r * Cfg::kPitch + 4 * (4 * ks + lq));
                }
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int n = 0; n < 4; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[n], acc[m][n], 0,
                                                                         0, 0);
            }
        }
    }

    if constexpr (MODE == kRowDot) {
        // per row: its 4 n-subtiles in order, the 16 lanes of a column group
        // by a fixed xor butterfly, then the two column waves in order
        __shared__ float red[2][kTile];
        const float* Af = reinterpret_cast<const float*>(A_);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = 64 * wm + 16 * m + 4 * lq + r;
                const float* arow = Af + (i0 + rl) * Kp + j0 + 64 * wn + l16;
                float v = 0.0f;
#pragma unroll
                for (int n = 0; n < 4; ++n) v += acc[m][n][r] * arow[16 * n];
#pragma unroll
                for (int msk = 8; msk >= 1; msk >>= 1) v += __shfl_xor(v, msk, 16);
                if (l16 == 0) red[wn][rl] = v;
            }
        __syncthreads();
        if (tid < kTile) part[(i0 + tid) * gridDim.x + bj] = red[0][tid] + red[1][tid];
        return;
    }
    // register r of lane l: row 4*(l/16)+r, column l%16 of each 16 x 16 tile
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int64_t j = j0 + 64 * wn + 16 * n + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = i0 + 64 * wm + 16 * m + 4 * lq + r;
                if (i >= I || j >= I) continue;
                if (bi == bj && i > j) continue;  // the pair is written from (j, i)
                const float v = acc[m][n][r];
                float* p = H + i * I + j;
                float* q = H + j * I + i;
                if (accumulate) {
                    const float nv = *p + v;
                    *p = nv;
                    if (i != j) *q = nv;
                } else {
                    *p = v;
                    if (i != j) *q = v;
                }
            }
        }
}

// ---- bf16: 256 x 256 tiles, operand stages through registers into LDS
constexpr int kBT = 256;                 // output tile
constexpr int kBThreads = 512;           // 8 waves: 2 (rows) x 4 (columns), 128 x 64 each
constexpr int kBK = 32;                  // tokens per stage (one MFMA step)
constexpr int kOpBytes = kBT * kBK * 2;  // one operand stage: 16 KB, 16 blocks of 1 KB
constexpr int kNBuf = 2;                 // stage slots in LDS
constexpr int kStrip = 8;                // tile rows per strip of the launch order

// Tile t of the upper triangle of an nb x nb tile grid, in strips of kStrip
// tile rows, each strip walked column by column (rows within a column).
__device__ __forceinline__ void tri_tile(int t, int nb, int& bi, int& bj) {
    int r0 = 0;
    for (;; r0 += kStrip) {  // strip r0: columns r0 .. nb-1, min(kStrip, c - r0 + 1) tiles each
        const int h = min(kStrip, nb - r0);
        // columns r0 .. r0+h-1 hold 1 .. h tiles, the nb - r0 - h after them h each
        const int n = h * (h + 1) / 2 + (nb - r0 - h) * h;
        if (t < n) break;
        t -= n;
    }
    const int h = min(kStrip, nb - r0);
    int c = r0;
    if (t < h * (h + 1) / 2) {
        while (t >= c - r0 + 1) {
            t -= c - r0 + 1;
            ++c;
        }
    } else {
        t -= h * (h + 1) / 2;
        c = r0 + h + t / h;
        t %= h;
    }
    bi = r0 + t;
    bj = c;
}

__global__ __launch_bounds__(kBThreads) void syrk_bf16_kernel(const uint16_t* __restrict__ Xt,
                                                              int64_t Tp, int64_t I, int nb,
                                                              int ntiles, int per,
                                                              float* __restrict__ H,
                                                              int accumulate) {
    // [stage slot][A, B][16 blocks of 1 KB]: block r16 holds, at lane
    // l = 16 lq + l16, the 8 tokens 8 lq .. 8 lq + 7 of the stage for row
    // 16 r16 + l16 of the operand's 256
    __shared__ __attribute__((aligned(16))) uint8_t st[kNBuf][2][kOpBytes];
    // consecutive block ids go to the 8 XCDs in turn: XCD x runs tiles
    // [x per, (x + 1) per) of the launch order
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= ntiles) return;  // uniform
    int bi, bj;
    tri_tile(t, nb, bi, bj);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l16 = lane & 15, lq = lane >> 4;
    const int64_t i0 = (int64_t)bi * kBT, j0 = (int64_t)bj * kBT;

    // wave w loads blocks 2w and 2w+1 of each operand; lane l of block b
    // reads the 16 bytes of row 16 b + l16 at token 8 lq of the stage
    const uint8_t* srcA[2];
    const uint8_t* srcB[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int64_t r = 16 * (2 * wave + q) + l16;
        srcA[q] = reinterpret_cast<const uint8_t*>(Xt + (i0 + r) * Tp + 8 * lq);
        srcB[q] = reinterpret_cast<const uint8_t*>(Xt + (j0 + r) * Tp + 8 * lq);
    }
    const int64_t nst = Tp / kBK;
    // a stage's 16 bytes per lane and block, in registers between its loads
    // and its stores into the stage's LDS slot.  Every step loads one stage,
    // so each wave always has the same number of loads in flight; stages
    // past the end re-read the last one (the last step stores one of them
    // into the slot not being read, which nobody reads again).
    struct Stage {
        u32x4_t v[4];
    };
    auto load = [&](int64_t sg, Stage& r) {
        const int64_t k0 = min(sg, nst - 1) * kBK * 2;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            r.v[q] = *reinterpret_cast<const u32x4_t*>(srcA[q] + k0);
            r.v[2 + q] = *reinterpret_cast<const u32x4_t*>(srcB[q] + k0);
        }
    };
    auto store = [&](int64_t sg, const Stage& r) {
        const int buf = (int)(sg % kNBuf);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int b = 2 * wave + q;
            reinterpret_cast<u32x4_t*>(st[buf][0] + 1024 * b)[lane] = r.v[q];
            reinterpret_cast<u32x4_t*>(st[buf][1] + 1024 * b)[lane] = r.v[2 + q];
        }
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Step s: stage s is in its LDS slot; the loads of stage s+2 are issued,
    // stage s is multiplied, and stage s+1 (loaded during step s-1) is stored
    // into the other slot.  The barrier at the top of each step makes the
    // stage stored in the step before visible, and keeps a slot from being
    // stored into while it is read (the other slot was last read in step
    // s-1).
    Stage r0, r1;
    load(0, r0);
    load(1, r1);
    store(0, r0);  // waits for stage 0's loads only: loads return in order
    auto step = [&](int64_t s0, Stage& nxt, Stage& nxt2) {
        // nxt holds stage s0+1 (in flight), nxt2 is free for stage s0+2
        lds_barrier();
        load(s0 + 2, nxt2);
        const int buf = (int)(s0 % kNBuf);
        const u32x4_t* As = reinterpret_cast<const u32x4_t*>(st[buf][0]) + lane;
        const u32x4_t* Bs = reinterpret_cast<const u32x4_t*>(st[buf][1]) + lane;
        u32x4_t a[8], b[4];
#pragma unroll
        for (int m = 0; m < 8; ++m) a[m] = As[64 * (8 * wm + m)];
#pragma unroll
        for (int n = 0; n < 4; ++n) b[n] = Bs[64 * (4 * wn + n)];
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, a[m]), __builtin_bit_cast(bf16x8_t, b[n]),
                    acc[m][n], 0, 0, 0);
        store(s0 + 1, nxt);
    };
    static_assert(kPadK % (2 * kBK) == 0, "an even number of stages");
    for (int64_t s0 = 0; s0 < nst; s0 += 2) {
        step(s0, r1, r0);
        step(s0 + 1, r0, r1);
    }

    // register r of lane l: row 4*(l/16)+r, column l%16 of each 16 x 16 tile
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int64_t j = j0 + 64 * wn + 16 * n + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = i0 + 128 * wm + 16 * m + 4 * lq + r;
                if (i >= I || j >= I) continue;
                if (bi == bj && i > j) continue;  // the pair is written from (j, i)
                const float v = acc[m][n][r];
                float* p = H + i * I + j;
                float* q = H + j * I + i;
                if (accumulate) {
                    const float nv = *p + v;
                    *p = nv;
                    if (i != j) *q = nv;
                } else {
                    *p = v;
                    if (i != j) *q = v;
                }
            }
        }
}

}  // namespace

int64_t hessian_full_rows(int64_t I) { return (I + kPadRows - 1) / kPadRows * kPadRows; }
int64_t hessian_full_tokens(int64_t T) { return (T + kPadK - 1) / kPadK * kPadK; }

hipError_t launch_hessian_full(const void* X, bool bf16, int64_t T, int64_t I, float* H,
                               int accumulate, void* workspace, hipStream_t s) {
    const int64_t Ip = hessian_full_rows(I), Tp = hessian_full_tokens(T);
    const dim3 tgrid((unsigned)(Tp / 64), (unsigned)(Ip / 64));
    const int64_t nb = Ip / kTile;
    if (nb > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nb, (unsigned)nb);
    if (bf16) {
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, tgrid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(X), T, I, Tp,
                           static_cast<uint16_t*>(workspace));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int nbb = (int)(Ip / kBT);
        const int ntiles = nbb * (nbb + 1) / 2;
        const int per = (ntiles + 7) / 8;
        hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)(8 * per)), dim3(kBThreads), 0, s,
                           static_cast<const uint16_t*>(workspace), Tp, I, nbb, ntiles, per, H,
                           accumulate);
    } else {
        hipLaunchKernelGGL(transpose_kernel<float>, tgrid, dim3(256), 0, s,
                           static_cast<const float*>(X), T, I, Tp,
                           static_cast<float*>(workspace));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((gemm_nt_kernel<false, kSymStore>), grid, dim3(kThreads), 0, s,
                           workspace, workspace, Tp, I, H, accumulate, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_rowdot_nt(const float* A, int64_t Mp, const float* B, int64_t Np, int64_t Kp,
                            float* part, hipStream_t s) {
    if (Mp % kTile || Np % kTile || Kp % SyrkCfg<false>::kK) return hipErrorInvalidValue;
    if (Mp / kTile > 65535 || Np / kTile > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(Np / kTile), (unsigned)(Mp / kTile));
    hipLaunchKernelGGL((gemm_nt_kernel<false, kRowDot>), grid, dim3(kThreads), 0, s, A, B, Kp,
                       (int64_t)0, nullptr, 0, part);
    return hipGetLastError();
}

}  // namespace qt
