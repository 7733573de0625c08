// The GPTQ column sweep with the int3-g64 rounder (the tt-stack issue page,
// pipeline table step 3: serial rounding inside 128-column blocks, then a
// matmul W[:, rest] -= E Hinv[blk, rest] carrying the block's scaled errors to
// every later column; Hinv is U, the upper Cholesky factor of the damped
// H^-1), and the terms of the page's proxy error tr(E H E^T) / tr(W H W^T).
//
// Sweep, per 128-column block:
//  * gptq_block_kernel: one lane per weight row (rows are independent), the
//    block's columns in two 64-column groups.  At a group's first column the
//    group scale is absmax/4 of its current values; then, column by column,
//    q = rne(w/s) clamped to [-4, 3] (IEEE division), err = (w - s q)/U[i][i]
//    and every later column of the group takes w_j = fma(-err, U[i][j], w_j).
//    The second group first takes the first group's updates in column order,
//    so every value sees exactly the operations of a plain column-by-column
//    sweep.  U's entries are the same for every lane (scalar loads).
//  * gptq_prop_kernel: Wc[:, b1:] -= Err[:, 0:128] U[b0:b1, b1:] on the f32
//    matrix cores (v_mfma_f32_16x16x4_f32, 128 x 128 output tiles).
#include <algorithm>

#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBlock = 128;  // sweep block (columns)
constexpr int kErrPitch = 68;  // LDS floats per lane of the first group's errors

constexpr int kUpitch = kBlock + 4;  // LDS floats per row of the U block

__device__ __forceinline__ float rne_code(float w, float s) {
    if (s == 0.0f) return 0.0f;
    const float q = __builtin_rintf(w / s);
    return fminf(fmaxf(q, -4.0f), 3.0f);
}

// One group of one row: at its first column the scale, then column by
// column the code, the scaled error and the updates of the later columns.
// Codes are collected four to a word; GI == 0 also leaves the errors in LDS
// for the block's second group.
template <int GI>
__device__ __forceinline__ float group_pass(float (&w)[kGroup], const float* ublk, float* er,
                                            float* elds, uint32_t (&qw)[kGroup / 4]) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) amax = fmaxf(amax, fabsf(w[j]));
    const float s = amax * 0.25f;
#pragma unroll
    for (int k = 0; k < kGroup / 4; ++k) qw[k] = 0u;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
        const float q = rne_code(w[i], s);
        const float t = s * q;
        const float r = w[i] - t;
        // keep each column's LDS reads next to their use
        asm volatile("" ::: "memory");
        const float* urow = ublk + i * kUpitch;
        const float e = r / urow[i];
        qw[i >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i & 3));
        er[i] = e;
        if (GI == 0) elds[i] = e;
#pragma unroll
        for (int j = i + 1; j < kGroup; ++j) w[j] = __builtin_fmaf(-e, urow[j], w[j]);
        // the updates happen in this column: left to the scheduler they sink
        // to their use and keep every loaded U value alive until then
#pragma unroll
        for (int j = i + 1; j < kGroup; ++j) asm volatile("" : "+v"(w[j]));
    }
    return s;
}

// Four waves (256 rows) per block, the block of columns [b0, min(b0+128, I)).
// U's 128 x 128 block sits in LDS, padded past I with 0 off the diagonal and
// 1 on it; padded columns hold w = 0, so their codes and errors are 0 and
// they change nothing (and are not stored).  Every row then runs one
// branch-free path.  vec: codes rows allow 16-byte stores (I % 16 == 0).
constexpr int kSweepRows = 256;

__global__ __launch_bounds__(kSweepRows) void gptq_block_kernel(
    float* __restrict__ Wc, int64_t O, int64_t I, const float* __restrict__ U, int64_t b0,
    float* __restrict__ scales, int8_t* __restrict__ codes, float* __restrict__ Err, int vec) {
    __shared__ __attribute__((aligned(16))) float Ub[kBlock * kUpitch];
    __shared__ __attribute__((aligned(16))) float errs[kSweepRows * kErrPitch];
    const int lane = threadIdx.x;
    if (vec && b0 + kBlock <= I) {
        // whole block inside U: 16-byte loads (I % 4 == 0 and b0 % 128 == 0)
        for (int p = lane; p < kBlock * kBlock / 4; p += kSweepRows) {
            const int i = p / (kBlock / 4), j4 = (p % (kBlock / 4)) * 4;
            *reinterpret_cast<float4*>(Ub + i * kUpitch + j4) =
                *reinterpret_cast<const float4*>(U + (b0 + i) * I + b0 + j4);
        }
    } else {
        for (int p = lane; p < kBlock * kBlock; p += kSweepRows) {
            const int i = p / kBlock, j = p % kBlock;
            const int64_t gi = b0 + i, gj = b0 + j;
            Ub[i * kUpitch + j] = (gi < I && gj < I) ? U[gi * I + gj] : (i == j ? 1.0f : 0.0f);
        }
    }
    __syncthreads();
    const int64_t o = (int64_t)blockIdx.x * kSweepRows + lane;
    if (o >= O) return;  // no cross-lane operations or barriers below
    const int64_t G = (I + kGroup - 1) / kGroup;
    const int64_t b1 = min(b0 + kBlock, I);
    float* wrow = Wc + o * I;
    float* elds = errs + lane * kErrPitch;
#pragma unroll 1
    for (int gi = 0; gi < 2; ++gi) {
        const int64_t c0 = b0 + kGroup * gi;
        if (c0 >= b1) break;
        const int n = (int)min<int64_t>(kGroup, b1 - c0);
        float w[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const float v = wrow[c0 + min(j, n - 1)];  // always inside the row
            w[j] = j < n ? v : 0.0f;
        }
        float* er = Err + o * kBlock + kGroup * gi;
        uint32_t qw[kGroup / 4];
        float s;
        if (gi == 0) {
            s = group_pass<0>(w, Ub, er, elds, qw);
        } else {
            // the first group's errors reach this group in column order
#pragma unroll 2
            for (int i = 0; i < kGroup; ++i) {
                asm volatile("" ::: "memory");
                const float e = elds[i];
                const float* urow = Ub + i * kUpitch + kGroup;
#pragma unroll
                for (int j = 0; j < kGroup; ++j) w[j] = __builtin_fmaf(-e, urow[j], w[j]);
#pragma unroll
                for (int j = 0; j < kGroup; ++j) asm volatile("" : "+v"(w[j]));
            }
            s = group_pass<1>(w, Ub + kGroup * kUpitch + kGroup, er, elds, qw);
        }
        scales[o * G + c0 / kGroup] = s;
        int8_t* cd = codes + o * I + c0;
        if (vec && n == kGroup) {
#pragma unroll
            for (int k = 0; k < kGroup / 16; ++k)
                reinterpret_cast<uint4*>(cd)[k] =
                    make_uint4(qw[4 * k], qw[4 * k + 1], qw[4 * k + 2], qw[4 * k + 3]);
        } else {
            for (int j = 0; j < n; ++j) {
                uint32_t word = 0u;
#pragma unroll
                for (int k = 0; k < kGroup / 4; ++k) word = (j >> 2) == k ? qw[k] : word;
                cd[j] = (int8_t)(word >> (8 * (j & 3)));
            }
        }
    }
}

// Wc[m][b1 + n] -= sum_k Err[m][k] U[b0 + k][b1 + n], k < 128, on 128 x 128
// tiles: 4 waves (2 x 2) of 64 x 64, the K range staged in two halves.
constexpr int kPT = 128;
constexpr int kPK = 64;                 // K per LDS stage
constexpr int kApitch = kPK + 4;        // floats per A row in LDS ([m][k])
constexpr int kBpitch = kPT + 4;        // floats per B row in LDS ([k][n])

__global__ __launch_bounds__(256) void gptq_prop_kernel(float* __restrict__ Wc, int64_t O,
                                                        int64_t I, const float* __restrict__ U,
                                                        int64_t b0,
                                                        const float* __restrict__ Err, int uvec) {
    __shared__ __attribute__((aligned(16))) float As[kPT * kApitch];
    __shared__ __attribute__((aligned(16))) float Bs[kPK * kBpitch];
    const int64_t b1 = b0 + kBlock;
    const int64_t N = I - b1;
    const int64_t m0 = (int64_t)blockIdx.y * kPT, n0 = (int64_t)blockIdx.x * kPT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, l16 = lane & 15, lq = lane >> 4;
    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int kh = 0; kh < kBlock; kh += kPK) {
        __syncthreads();
        // A: 128 rows x 64 k (16-byte pieces); B: 64 k x 128 n (scalars)
        for (int p = tid; p < kPT * kPK / 4; p += 256) {
            const int r = p / (kPK / 4), c4 = (p % (kPK / 4)) * 4;
            const int64_t m = m0 + r;
            f32x4_t v = {0.f, 0.f, 0.f, 0.f};
            if (m < O) v = *reinterpret_cast<const f32x4_t*>(Err + m * kBlock + kh + c4);
            *reinterpret_cast<f32x4_t*>(As + r * kApitch + c4) = v;
        }
        if (uvec && n0 + kPT <= N) {  // 16-byte loads: I % 4 == 0, whole tile inside
            for (int p = tid; p < kPK * kPT / 4; p += 256) {
                const int k = p / (kPT / 4), c4 = (p % (kPT / 4)) * 4;
                *reinterpret_cast<f32x4_t*>(Bs + k * kBpitch + c4) =
                    *reinterpret_cast<const f32x4_t*>(U + (b0 + kh + k) * I + b1 + n0 + c4);
            }
        } else {
            for (int p = tid; p < kPK * kPT; p += 256) {
                const int k = p / kPT, c = p % kPT;
                const int64_t nn = n0 + c;
                Bs[k * kBpitch + c] = nn < N ? U[(b0 + kh + k) * I + b1 + nn] : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll 4
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
            if (nn >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t mm = m0 + 64 * wm + 16 * m + 4 * lq + r;
                if (mm < O) {
                    float* p = Wc + mm * I + b1 + nn;
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
    return (size_t)(err_offset(O, I) + O * kBlock) * sizeof(float);
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
    for (int64_t b0 = 0; b0 < I; b0 += kBlock) {
        hipLaunchKernelGGL(gptq_block_kernel, dim3(rb), dim3(kSweepRows), 0, s, Wc, O, I, U, b0,
                           scales, codes, Err, vec);
        const int64_t rest = I - (b0 + kBlock);
        if (rest > 0) {
            const dim3 grid((unsigned)((rest + kPT - 1) / kPT), (unsigned)((O + kPT - 1) / kPT));
            hipLaunchKernelGGL(gptq_prop_kernel, grid, dim3(256), 0, s, Wc, O, I, U, b0, Err,
                               uvec);
        }
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
