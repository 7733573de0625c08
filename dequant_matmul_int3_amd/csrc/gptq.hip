// The GPTQ column sweep with the int3-g64 rounder (the tt-stack issue page,
// pipeline table step 3: serial rounding inside 128-column blocks, then a
// matmul W[:, rest] -= E Hinv[blk, rest] carrying the block's scaled errors to
// every later column; Hinv is U, the upper Cholesky factor of the damped
// H^-1), and the terms of the page's proxy error tr(E H E^T) / tr(W H W^T).
//
// Sweep, per 128-column block:
//  * gptq_block_kernel: four lanes per weight row (rows are independent), each
//    lane 16 columns of each of the block's two 64-column groups.  At a
//    group's first column the group scale is absmax/4 of its current values;
//    then, column by column, the lane owning the column forms
//    q = rne(w/s) clamped to [-4, 3] (IEEE division) and err = (w - s q)/U[i][i],
//    broadcasts err to its quad, and every later column of the group takes
//    w_j = fma(-err, U[i][j], w_j).  The second group first takes the first
//    group's updates in column order, so every value sees exactly the
//    operations of a plain column-by-column sweep.
//  * gptq_prop_kernel: the block's scaled errors reach the later columns,
//    Wc[:, later] -= Err U[block, later], on the f32 matrix cores
//    (v_mfma_f32_16x16x4_f32, 128 x 128 output tiles).  Blocks are grouped
//    four to a 512-column super-block: a block updates only the rest of its
//    super-block, and once the super-block is done one rank-512 product
//    carries all four blocks' errors to every column after it (the same sums
//    in another grouping; a quarter of the passes over the trailing weights).
#include <algorithm>

#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBlock = 128;  // sweep block (columns)
constexpr int kSuper = 512;  // blocks whose updates of later columns are deferred together

constexpr int kUpitch = kBlock + 4;  // LDS floats per row of the U block

__device__ __forceinline__ float rne_code(float w, float s) {
    if (s == 0.0f) return 0.0f;
    const float q = __builtin_rintf(w / s);
    return fminf(fmaxf(q, -4.0f), 3.0f);
}

// Four lanes share a row (a DPP quad); lane t of the quad owns columns
// [16 t, 16 t + 16) of each 64-column group.
constexpr int kQ = 4;                // lanes per row
constexpr int kQC = kGroup / kQ;     // columns per lane and group

// value of quad lane S, in every lane of the quad (S folds to a constant
// inside the unrolled column loops)
__device__ __forceinline__ float quad_bcast(float v, int S) {
    const int b = __float_as_int(v);
    int r;
    switch (S) {
        case 0: r = __builtin_amdgcn_update_dpp(0, b, 0x00, 0xF, 0xF, false); break;
        case 1: r = __builtin_amdgcn_update_dpp(0, b, 0x55, 0xF, 0xF, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, b, 0xAA, 0xF, 0xF, false); break;
        default: r = __builtin_amdgcn_update_dpp(0, b, 0xFF, 0xF, 0xF, false); break;
    }
    return __int_as_float(r);
}

// One group of one row: at its first column the scale (absmax/4 over the
// quad), then column by column the owner lane's code and scaled error, sent
// to the quad, and every lane's update of its columns.  Updates of columns at
// or before the current one multiply U's zeros (or reach a column already
// coded), so every lane runs the same straight-line code; a later column
// still takes exactly fma(-err_i, U[i][j], w_j) for i = 0, 1, ... in order.
// ublk: the U block rows of this group's columns, offset to this group's
// first column; qw collects the lane's codes four to a word, eown its errors.
__device__ __forceinline__ float group_pass(float (&w)[kQC], const float* ublk, int t,
                                            uint32_t (&qw)[kQC / 4], float (&eown)[kQC]) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kQC; ++j) amax = fmaxf(amax, fabsf(w[j]));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1,
                                                                  0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E,
                                                                  0xF, 0xF, false)));
    const float s = amax * 0.25f;
#pragma unroll
    for (int k = 0; k < kQC / 4; ++k) qw[k] = 0u;
    const float* ucol = ublk + kQC * t;  // this lane's columns
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
        const int owner = i / kQC, li = i % kQC;
        // keep each column's LDS reads next to their use
        asm volatile("" ::: "memory");
        const float q = rne_code(w[li], s);  // meaningful in the owner lane
        const float tq = s * q;
        const float r = w[li] - tq;
        const float e = quad_bcast(r / ublk[i * kUpitch + i], owner);
        if (t == owner) {
            qw[li >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (li & 3));
            eown[li] = e;
        }
        const float* urow = ucol + i * kUpitch;
#pragma unroll
        for (int j = 0; j < kQC; ++j) w[j] = __builtin_fmaf(-e, urow[j], w[j]);
        // the updates happen in this column: left to the scheduler they sink
        // to their use and keep every loaded U value alive until then
#pragma unroll
        for (int j = 0; j < kQC; ++j) asm volatile("" : "+v"(w[j]));
    }
    return s;
}

// 64 rows (16 per wave, four lanes each) per block, the block of columns
// [b0, min(b0+128, I)).  U's 128 x 128 block sits in LDS with zeros below the
// diagonal, padded past I with 0 off the diagonal and 1 on it; padded columns
// hold w = 0, so their codes and errors are 0 and they change nothing (and
// are not stored).  vec: code rows allow 16-byte stores (I % 16 == 0) and
// weight rows 16-byte loads.
constexpr int kSweepThreads = 256;
constexpr int kSweepRows = kSweepThreads / kQ;

__global__ __launch_bounds__(kSweepThreads) void gptq_block_kernel(
    float* __restrict__ Wc, int64_t O, int64_t I, const float* __restrict__ U, int64_t b0,
    float* __restrict__ scales, int8_t* __restrict__ codes, float* __restrict__ Err, int64_t eoff,
    int vec) {
    __shared__ __attribute__((aligned(16))) float Ub[kBlock * kUpitch];
    const int tid = threadIdx.x;
    if (vec && b0 + kBlock <= I) {
        // whole block inside U: 16-byte loads (I % 4 == 0 and b0 % 128 == 0)
        for (int p = tid; p < kBlock * kBlock / 4; p += kSweepThreads) {
            const int i = p / (kBlock / 4), j4 = (p % (kBlock / 4)) * 4;
            float4 v = *reinterpret_cast<const float4*>(U + (b0 + i) * I + b0 + j4);
            if (j4 + 0 < i) v.x = 0.0f;
            if (j4 + 1 < i) v.y = 0.0f;
            if (j4 + 2 < i) v.z = 0.0f;
            if (j4 + 3 < i) v.w = 0.0f;
            *reinterpret_cast<float4*>(Ub + i * kUpitch + j4) = v;
        }
    } else {
        for (int p = tid; p < kBlock * kBlock; p += kSweepThreads) {
            const int i = p / kBlock, j = p % kBlock;
            const int64_t gi = b0 + i, gj = b0 + j;
            Ub[i * kUpitch + j] =
                j < i ? 0.0f : ((gi < I && gj < I) ? U[gi * I + gj] : (i == j ? 1.0f : 0.0f));
        }
    }
    __syncthreads();
    // rows past O compute on row O - 1's values and store nothing; all lanes
    // stay for the quad broadcasts
    const int t = tid & (kQ - 1);
    const int64_t o = (int64_t)blockIdx.x * kSweepRows + tid / kQ;
    const bool live = o < O;
    const int64_t orow = live ? o : O - 1;
    const int64_t G = (I + kGroup - 1) / kGroup;
    const int64_t b1 = min(b0 + kBlock, I);
    const float* wrow = Wc + orow * I;
    float e0[kQC];  // the first group's errors of this lane's columns
#pragma unroll 1
    for (int gi = 0; gi < 2; ++gi) {
        const int64_t c0 = b0 + kGroup * gi;
        if (c0 >= b1) break;  // uniform
        const int n = (int)min<int64_t>(kGroup, b1 - c0);
        const int cl = kQC * t;  // this lane's first column in the group
        float w[kQC];
        if (vec && n == kGroup) {
#pragma unroll
            for (int k = 0; k < kQC / 4; ++k) {
                const float4 v = *reinterpret_cast<const float4*>(wrow + c0 + cl + 4 * k);
                w[4 * k] = v.x;
                w[4 * k + 1] = v.y;
                w[4 * k + 2] = v.z;
                w[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kQC; ++j) {
                const float v = wrow[c0 + min(cl + j, n - 1)];  // always inside the row
                w[j] = cl + j < n ? v : 0.0f;
            }
        }
        uint32_t qw[kQC / 4];
        float eown[kQC];
        float s;
        if (gi == 0) {
            s = group_pass(w, Ub, t, qw, eown);
#pragma unroll
            for (int j = 0; j < kQC; ++j) e0[j] = eown[j];
        } else {
            // the first group's errors reach this group in column order
            const float* ucol = Ub + kGroup + cl;
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                asm volatile("" ::: "memory");
                const float e = quad_bcast(e0[i % kQC], i / kQC);
                const float* urow = ucol + i * kUpitch;
#pragma unroll
                for (int j = 0; j < kQC; ++j) w[j] = __builtin_fmaf(-e, urow[j], w[j]);
#pragma unroll
                for (int j = 0; j < kQC; ++j) asm volatile("" : "+v"(w[j]));
            }
            s = group_pass(w, Ub + kGroup * kUpitch + kGroup, t, qw, eown);
        }
        if (!live) continue;
        if (t == 0) scales[o * G + c0 / kGroup] = s;
        float* er = Err + o * kSuper + eoff + kGroup * gi + cl;
        int8_t* cd = codes + o * I + c0 + cl;
        if (vec && n == kGroup) {
#pragma unroll
            for (int k = 0; k < kQC / 4; ++k)
                reinterpret_cast<float4*>(er)[k] =
                    make_float4(eown[4 * k], eown[4 * k + 1], eown[4 * k + 2], eown[4 * k + 3]);
            *reinterpret_cast<uint4*>(cd) = make_uint4(qw[0], qw[1], qw[2], qw[3]);
        } else {
#pragma unroll
            for (int j = 0; j < kQC; ++j) {
                if (cl + j < n) {
                    er[j] = eown[j];
                    cd[j] = (int8_t)(qw[j >> 2] >> (8 * (j & 3)));
                }
            }
        }
    }
}

// Wc[m][c] -= sum_{k < kw} Err[m][eo + k] U[kb + k][c] for m < O and
// c0 <= c < cend, on 128 x 128 tiles: 4 waves (2 x 2) of 64 x 64, K staged
// through LDS 32 at a time with the next stage loaded into registers while
// the current one is multiplied.  Err rows have pitch kSuper.  uvec: U rows
// allow 16-byte loads (I % 4 == 0, U 16-byte aligned).
constexpr int kPT = 128;
constexpr int kPK = 32;                 // K per LDS stage
constexpr int kApitch = kPK + 4;        // floats per A row in LDS ([m][k])
constexpr int kBpitch = kPT + 4;        // floats per B row in LDS ([k][n])
constexpr int kPL = kPT * kPK / 4 / 256;  // 16-byte pieces per thread and operand (4)

__global__ __launch_bounds__(256) void gptq_prop_kernel(float* __restrict__ Wc, int64_t O,
                                                        int64_t I, const float* __restrict__ U,
                                                        int64_t kb, int kw,
                                                        const float* __restrict__ Err, int64_t eo,
                                                        int64_t c0, int64_t cend, int uvec) {
    __shared__ __attribute__((aligned(16))) float As[kPT * kApitch];
    __shared__ __attribute__((aligned(16))) float Bs[kPK * kBpitch];
    const int64_t m0 = (int64_t)blockIdx.y * kPT, n0 = c0 + (int64_t)blockIdx.x * kPT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, l16 = lane & 15, lq = lane >> 4;
    const bool bvec = uvec && n0 + kPT <= cend;  // uniform
    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // A: 128 rows x 32 k, piece p = row p / 8, k 4 (p % 8); B: 32 k x 128 n,
    // piece p = k p / 32, n 4 (p % 32); zeros outside the operands
    f32x4_t ra[kPL], rb[kPL];
    auto load = [&](int k0) {
#pragma unroll
        for (int l = 0; l < kPL; ++l) {
            const int p = tid + 256 * l;
            {
                const int r = p / (kPK / 4), k4 = (p % (kPK / 4)) * 4;
                const int64_t m = m0 + r;
                f32x4_t v = {0.f, 0.f, 0.f, 0.f};
                if (m < O && k0 + k4 < kw)  // kw % 4 == 0
                    v = *reinterpret_cast<const f32x4_t*>(Err + m * kSuper + eo + k0 + k4);
                ra[l] = v;
            }
            {
                const int k = p / (kPT / 4), c4 = (p % (kPT / 4)) * 4;
                const int64_t ur = kb + k0 + k, c = n0 + c4;
                f32x4_t v = {0.f, 0.f, 0.f, 0.f};
                if (k0 + k < kw) {
                    if (bvec) {
                        v = *reinterpret_cast<const f32x4_t*>(U + ur * I + c);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (c + q < cend) v[q] = U[ur * I + c + q];
                    }
                }
                rb[l] = v;
            }
        }
    };
    load(0);
    for (int k0 = 0; k0 < kw; k0 += kPK) {
        __syncthreads();  // the previous stage is consumed
#pragma unroll
        for (int l = 0; l < kPL; ++l) {
            const int p = tid + 256 * l;
            *reinterpret_cast<f32x4_t*>(As + (p / (kPK / 4)) * kApitch + (p % (kPK / 4)) * 4) =
                ra[l];
            *reinterpret_cast<f32x4_t*>(Bs + (p / (kPT / 4)) * kBpitch + (p % (kPT / 4)) * 4) =
                rb[l];
        }
        __syncthreads();
        if (k0 + kPK < kw) load(k0 + kPK);  // the next stage in flight
#pragma unroll
        for (int ks = 0; ks < kPK / 4; ++ks) {
            float a[4], b[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) a[m] = As[(64 * wm + 16 * m + l16) * kApitch + 4 * ks + lq];
#pragma unroll
            for (int n = 0; n < 4; ++n) b[n] = Bs[(4 * ks + lq) * kBpitch + 64 * wn + 16 * n + l16];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[n], acc[m][n], 0, 0, 0);
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int64_t nn = n0 + 64 * wn + 16 * n + l16;
            if (nn >= cend) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t mm = m0 + 64 * wm + 16 * m + 4 * lq + r;
                if (mm < O) {
                    float* p = Wc + mm * I + nn;
                    *p = *p - acc[m][n][r];
                }
            }
        }
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src, int64_t n,
                                                       float* __restrict__ dst) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

// ---------------------------------------------------------------- proxy
// R = [W; E] padded to [Mp x Kp] (E = W - s v decoded from the packed
// planes), H padded to [Kp x Kp]; zeros outside.
__global__ __launch_bounds__(256) void proxy_prep_kernel(const float* __restrict__ W,
                                                         const uint8_t* __restrict__ packed,
                                                         const float* __restrict__ scales,
                                                         int64_t O, int64_t I, int64_t Kp,
                                                         float* __restrict__ R) {
    const int64_t row = blockIdx.y;  // 0 .. Mp-1
    const int64_t G = (I + kGroup - 1) / kGroup;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < Kp;
         k += (int64_t)gridDim.x * 256) {
        float v = 0.0f;
        const int64_t o = row < O ? row : row - O;
        if (o < O && k < I) {
            const float w = W[o * I + k];
            if (row < O) {
                v = w;
            } else {
                const int64_t g = k / kGroup;
                const int j = (int)(k % kGroup);
                const uint8_t* gp = packed + (o * G + g) * kGroupBytes;
                const int lo = (gp[j >> 2] >> (2 * (j & 3))) & 3;
                const int hi = (gp[16 + (j >> 3)] >> (j & 7)) & 1;
                const float code = (float)((lo | (hi << 2)) - 4);
                v = w - scales[o * G + g] * code;
            }
        }
        R[row * Kp + k] = v;
    }
}

__global__ __launch_bounds__(256) void pad_square_kernel(const float* __restrict__ H, int64_t I,
                                                         int64_t Kp, float* __restrict__ Hp) {
    const int64_t r = blockIdx.y;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < Kp;
         k += (int64_t)gridDim.x * 256)
        Hp[r * Kp + k] = (r < I && k < I) ? H[r * I + k] : 0.0f;
}

// Per row of R: the partials of its column tiles in order, then the W rows
// and the E rows, each in row order, in f64.
__global__ __launch_bounds__(256) void proxy_reduce_kernel(const float* __restrict__ part,
                                                           int64_t O, int64_t ntiles,
                                                           double* __restrict__ terms) {
    __shared__ double sums[2][256];
    for (int h = 0; h < 2; ++h) {
        double s = 0.0;
        for (int64_t o = threadIdx.x; o < O; o += 256) {
            const float* p = part + (h * O + o) * ntiles;
            double r = 0.0;
            for (int64_t t = 0; t < ntiles; ++t) r += (double)p[t];
            s += r;
        }
        sums[h][threadIdx.x] = s;
    }
    __syncthreads();
    for (int m = 128; m >= 1; m >>= 1) {
        if ((int)threadIdx.x < m) {
            sums[0][threadIdx.x] += sums[0][threadIdx.x + m];
            sums[1][threadIdx.x] += sums[1][threadIdx.x + m];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        terms[0] = sums[1][0];  // tr(E H E^T)
        terms[1] = sums[0][0];  // tr(W H W^T)
    }
}

}  // namespace

// The current weights, then (16-byte aligned) the block errors.
static int64_t err_offset(int64_t O, int64_t I) { return (O * I + 3) / 4 * 4; }

size_t gptq_workspace(int64_t O, int64_t I) {
    return (size_t)(err_offset(O, I) + O * kSuper) * sizeof(float);
}

hipError_t launch_gptq_i3(const float* W, int64_t O, int64_t I, const float* U, float* scales,
                          int8_t* codes, void* workspace, hipStream_t s) {
    float* Wc = static_cast<float*>(workspace);
    float* Err = Wc + err_offset(O, I);
    const int64_t nel = O * I;
    hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)std::min<int64_t>((nel + 255) / 256, 65536)),
                       dim3(256), 0, s, W, nel, Wc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned rb = (unsigned)((O + kSweepRows - 1) / kSweepRows);
    // 16-byte code stores need I % 16 == 0; 16-byte U loads need I % 4 == 0
    const int vec = (I % 16 == 0) && ((reinterpret_cast<uintptr_t>(codes) & 15) == 0) &&
                    ((reinterpret_cast<uintptr_t>(U) & 15) == 0);
    const int uvec = (I % 4 == 0) && ((reinterpret_cast<uintptr_t>(U) & 15) == 0);
    auto prop = [&](int64_t kb, int kw, int64_t eo, int64_t c0, int64_t cend) {
        if (cend <= c0) return;
        const dim3 grid((unsigned)((cend - c0 + kPT - 1) / kPT), (unsigned)((O + kPT - 1) / kPT));
        hipLaunchKernelGGL(gptq_prop_kernel, grid, dim3(256), 0, s, Wc, O, I, U, kb, kw, Err, eo,
                           c0, cend, uvec);
    };
    for (int64_t S0 = 0; S0 < I; S0 += kSuper) {
        const int64_t S1 = std::min<int64_t>(S0 + kSuper, I);
        for (int64_t b0 = S0; b0 < S1; b0 += kBlock) {
            hipLaunchKernelGGL(gptq_block_kernel, dim3(rb), dim3(kSweepThreads), 0, s, Wc, O, I, U,
                               b0, scales, codes, Err, b0 - S0, vec);
            // the rest of the super-block; a short last block has no columns after it
            if (b0 + kBlock < S1) prop(b0, kBlock, b0 - S0, b0 + kBlock, S1);
        }
        // every column after the super-block, from all of its blocks (a short
        // last super-block has no columns after it, so kw is a whole kSuper)
        if (S1 < I) prop(S0, kSuper, 0, S1, I);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int64_t proxy_pad(int64_t n) { return (n + 127) / 128 * 128; }

size_t gptq_proxy_workspace(int64_t O, int64_t I) {
    const int64_t Mp = proxy_pad(2 * O), Kp = proxy_pad(I);
    return (size_t)(Mp * Kp + Kp * Kp + Mp * (Kp / 128)) * sizeof(float);
}

hipError_t launch_gptq_proxy(const float* W, const uint8_t* packed, const float* scales,
                             int64_t O, int64_t I, const float* H, double* terms,
                             void* workspace, hipStream_t s) {
    const int64_t Mp = proxy_pad(2 * O), Kp = proxy_pad(I);
    float* R = static_cast<float*>(workspace);
    float* Hp = R + Mp * Kp;
    float* part = Hp + Kp * Kp;
    const unsigned cols = (unsigned)std::min<int64_t>((Kp + 255) / 256, 64);
    if (Mp > 65535 || Kp > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(proxy_prep_kernel, dim3(cols, (unsigned)Mp), dim3(256), 0, s, W, packed,
                       scales, O, I, Kp, R);
    hipLaunchKernelGGL(pad_square_kernel, dim3(cols, (unsigned)Kp), dim3(256), 0, s, H, I, Kp,
                       Hp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_rowdot_nt(R, Mp, Hp, Kp, Kp, part, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proxy_reduce_kernel, dim3(1), dim3(256), 0, s, part, O, Kp / 128, terms);
    return hipGetLastError();
}

}  // namespace qt
