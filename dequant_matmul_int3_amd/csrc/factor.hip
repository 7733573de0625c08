// The GPTQ factor on the device: U = the upper Cholesky factor of A^-1,
// A = H + damp * mean(diag H) * I (the tt-stack issue page, pipeline table
// step 2: a Cholesky / inverse of H, there on the host with LAPACK, "blocked
// Cholesky on device later").
//
// With J the reversal, J A J = C C^T (C lower); then U = J C^-1 J is upper
// with U^T U = A^-1.  Everything runs in f64 (tile products on the f64 matrix
// cores, the rest on the vector ALUs), in 64-wide panels:
//   Cholesky, right-looking: factor the diagonal block in LDS, solve the
//   panel below it row by row, subtract the panel's outer product from the
//   trailing lower triangle (128 x 128 tiles);
//   inverse, recursively: every 64 x 64 diagonal block at once, then level
//   by level [[A, 0], [B, D]]^-1 = [[A^-1, 0], [-D^-1 B A^-1, D^-1]] for all
//   pairs of a level at once (two batched tile products through a scratch
//   buffer; the triangular factors' zero halves are skipped).
// A non-positive pivot sets *info to its 1-based column (of the reversed
// matrix) and is replaced by 1 so that every later step stays finite.
#include <algorithm>

#include "qt_internal.h"

namespace qt {
namespace {

constexpr int kNB = 64;      // panel width of the diagonal factorization
constexpr int kOuter = 512;  // columns per rank-k trailing update

// mean(diag H) * damp, summed in f64 in a fixed order by one block.
__global__ __launch_bounds__(256) void damp_kernel(const float* __restrict__ H, int64_t n,
                                                   double damp, double* __restrict__ add,
                                                   int32_t* __restrict__ info) {
    __shared__ double part[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)H[i * n + i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int m = 128; m >= 1; m >>= 1) {
        if ((int)threadIdx.x < m) part[threadIdx.x] += part[threadIdx.x + m];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *add = damp * (part[0] / (double)n);
        *info = 0;
    }
}

// B[i][j] = A[n-1-i][n-1-j] in f64, lower triangle (j <= i) only.
__global__ __launch_bounds__(256) void reverse_kernel(const float* __restrict__ H, int64_t n,
                                                      const double* __restrict__ add,
                                                      double* __restrict__ B) {
    const int64_t i = blockIdx.y;
    const double a = *add;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j <= i && j < n;
         j += (int64_t)gridDim.x * 256) {
        double v = (double)H[(n - 1 - i) * n + (n - 1 - j)];
        if (i == j) v += a;
        B[i * n + j] = v;
    }
}

// Cholesky of one kNB x kNB diagonal block in place (lower triangle), four
// waves: lane i holds row i, wave w its columns 16w .. 16w+15 (zeros above
// the diagonal).  Blocked by 16-column panels: the panel's wave factors it
// alone (each pivot and column entry read from its lane with readlane),
// writes it to LDS, and after a barrier the waves right of it subtract the
// panel's rank-16 product from their columns; every entry's updates still
// run over the columns in order.  Columns past kb (the last, narrower block)
// are zero rows and columns: a unit pivot there changes nothing that is
// stored, and so does a non-positive pivot, which also sets *info.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ B, int64_t n,
                                                         int64_t k0, int kb,
                                                         int32_t* __restrict__ info) {
    constexpr int kPW = 16;  // panel width: one wave's columns
    __shared__ double pan[kNB][kPW + 1];
    const int i = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j0 = kPW * w;
    const double* row = B + (k0 + min(i, kb - 1)) * n + k0;
    double x[kPW];
#pragma unroll
    for (int jl = 0; jl < kPW; ++jl) {
        const int j = j0 + jl;
        const double v = row[min(j, kb - 1)];  // inside the block
        x[jl] = (i < kb && j < kb && j <= i) ? v : 0.0;
    }
    for (int p = 0; p < kNB / kPW; ++p) {
        if (w == p) {  // uniform over the wave
#pragma unroll
            for (int cl = 0; cl < kPW; ++cl) {
                const int c = j0 + cl;
                double d = readlane_f64(x[cl], c);
                if (c >= kb) {  // uniform
                    d = 1.0;
                } else if (!(d > 0.0)) {  // uniform
                    if (i == 0 && *info == 0) *info = (int32_t)(k0 + c + 1);
                    d = 1.0;
                }
                // 1/sqrt(d): the hardware estimate and one Newton step
                // (doubling its correct bits), then sqrt(d) = d / sqrt(d)
                const double r0 = __builtin_amdgcn_rsq(d);
                const double res = __builtin_fma(-d * r0, r0, 1.0);
                const double rs = __builtin_fma(0.5 * r0, res, r0);
                x[cl] = i == c ? d * rs : (i > c ? x[cl] * rs : x[cl]);
#pragma unroll
                for (int jl = cl + 1; jl < kPW; ++jl)
                    x[jl] = __builtin_fma(-x[cl], readlane_f64(x[cl], j0 + jl), x[jl]);
            }
#pragma unroll
            for (int cl = 0; cl < kPW; ++cl) pan[i][cl] = x[cl];
        }
        __syncthreads();
        if (w > p) {
#pragma unroll
            for (int cl = 0; cl < kPW; ++cl) {
                const double a = pan[i][cl];
#pragma unroll
                for (int jl = 0; jl < kPW; ++jl)
                    x[jl] = __builtin_fma(-a, pan[j0 + jl][cl], x[jl]);
            }
        }
        __syncthreads();  // the panel is read before the next one is written
    }
    if (i < kb) {
        double* out = B + (k0 + i) * n + k0;
#pragma unroll
        for (int jl = 0; jl < kPW; ++jl) {
            const int j = j0 + jl;
            if (j < kb && j <= i) out[j] = x[jl];
        }
    }
}

// DPP quad move of an f64 value (two 32-bit moves), CTRL a quad_perm: 0xB1
// gives lane l the value of lane l ^ 1, 0x4E of lane l ^ 2, 0x55 * S of lane S.
template <int CTRL>
__device__ __forceinline__ double quad_dpp(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFFll), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double quad_bcast(double v, int S) {  // S folds to a constant
    switch (S) {
        case 0: return quad_dpp<0x00>(v);
        case 1: return quad_dpp<0x55>(v);
        case 2: return quad_dpp<0xAA>(v);
        default: return quad_dpp<0xFF>(v);
    }
}

// Rows below the diagonal block: x C_kk^T = b by forward substitution over
// the columns, four lanes per row (a DPP quad): lane t keeps the entries
// 4k + t of the row (the right-hand side b, and the solution x, zero until
// solved), sums its terms of each column, the quad adds its four partial
// sums in a fixed order and every lane forms the column's x.  Terms at or
// right of the column multiply the triangle's zeros or an unsolved zero, so
// no lane branches.  The diagonal's reciprocals are formed once per block
// (LDS holds -L below the diagonal, so the sums need no negation); 16 rows
// per block.
__global__ __launch_bounds__(64) void trsm_panel_kernel(double* __restrict__ B, int64_t n,
                                                        int64_t k0) {
    __shared__ double L[kNB][kNB + 1];
    __shared__ double rdiag[kNB];
    {
        // thread i stages row i of the diagonal block: all of its loads are
        // issued before the first is used (one latency, not one per entry)
        const int i = threadIdx.x;
        const double* src = B + (k0 + i) * n + k0;
        double v[kNB];
#pragma unroll
        for (int j = 0; j < kNB; ++j) v[j] = src[j];
        double d = 1.0;
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            L[i][j] = j < i ? -v[j] : 0.0;
            d = j == i ? v[j] : d;
        }
        rdiag[i] = 1.0 / d;
    }
    __syncthreads();
    constexpr int kQK = kNB / 4;
    const int t = threadIdx.x & 3;
    const int64_t r = k0 + kNB + (int64_t)blockIdx.x * 16 + (threadIdx.x >> 2);
    const bool live = r < n;  // rows past n run on row n - 1 and store nothing
    double* row = B + (live ? r : n - 1) * n + k0;
    double bx[kQK], xs[kQK];
#pragma unroll
    for (int k = 0; k < kQK; ++k) {
        bx[k] = row[4 * k + t];
        xs[k] = 0.0;
    }
#pragma unroll
    for (int c = 0; c < kNB; ++c) {
        double part = 0.0;
#pragma unroll
        for (int k = 0; k <= c / 4; ++k) part = __builtin_fma(xs[k], L[c][4 * k + t], part);
        // quad sum in a fixed order: (p0 + p1) + (p2 + p3) in every lane
        part += quad_dpp<0xB1>(part);
        part += quad_dpp<0x4E>(part);
        const double xc = (quad_bcast(bx[c / 4], c % 4) + part) * rdiag[c];
        xs[c / 4] = t == c % 4 ? xc : xs[c / 4];
    }
    if (live) {
#pragma unroll
        for (int k = 0; k < kQK; ++k) row[4 * k + t] = xs[k];
    }
}

// ---------------------------------------------------------------- f64 tiles
// Tile products on the f64 matrix cores (v_mfma_f64_16x16x4_f64, the same
// rate as the f64 vector ALUs but one LDS operand read per 16 products instead
// of one per 4): a TILE x TILE output tile, 4 waves as 2 x 2 of (TILE/2)^2,
// K staged through LDS kKC at a time as [row][k] with a 17-double pitch (the
// operand reads of a half-wave and the staging stores hit distinct banks).
// acc[m][n][r] of lane l is row (TILE/2) wm + 16 m + l/16 + 4 r, column
// (TILE/2) wn + 16 n + l%16 of the tile (the instruction's result layout).
// acc += sum_k P(row, k) Q(k, col) for k in [kbeg, kend); P and Q come from
// loaders that return 0 outside their operand.  QT: Q's memory is [col][k]
// (k contiguous), so its loads walk k like P's.
typedef __attribute__((ext_vector_type(4))) double f64x4_t;
constexpr int kKC = 16;
constexpr int kKP = kKC + 1;

template <int TILE>
struct TileAcc {
    static constexpr int MT = TILE / 32;  // 16 x 16 products per wave and dimension
    f64x4_t v[MT][MT];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < MT; ++n) v[m][n] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    }
    // f(row, col, value) for every element this lane holds
    template <typename F>
    __device__ __forceinline__ void each(F f) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int rb = (TILE / 2) * (wave >> 1) + (lane >> 4), cb = (TILE / 2) * (wave & 1) + (lane & 15);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) f(rb + 16 * m + 4 * r, cb + 16 * n, v[m][n][r]);
    }
};

template <int TILE, bool QT = false, typename LP, typename LQ>
__device__ __forceinline__ void tile_product(int64_t kbeg, int64_t kend, LP ldp, LQ ldq,
                                             TileAcc<TILE>& acc, double (*Ps)[kKP],
                                             double (*Qs)[kKP]) {
    constexpr int MT = TileAcc<TILE>::MT;
    constexpr int NL = kKC * TILE / 256;  // staged values per thread and operand
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ra = (TILE / 2) * (wave >> 1) + (lane & 15), ca = (TILE / 2) * (wave & 1) + (lane & 15);
    const int lq = lane >> 4;
    // staging: P(r, k) with consecutive threads walking k (row-major
    // operands), Q(k, c) walking c (or k when QT)
    double pv[NL], qv[NL];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int p = tid + 256 * l;
            {
                const int kk = p % kKC, r = p / kKC;
                const int64_t k = k0 + kk;
                pv[l] = k < kend ? ldp(r, k) : 0.0;
            }
            {
                const int c = QT ? p / kKC : p % TILE, kk = QT ? p % kKC : p / TILE;
                const int64_t k = k0 + kk;
                qv[l] = k < kend ? ldq(k, c) : 0.0;
            }
        }
    };
    if (kbeg < kend) load(kbeg);
    for (int64_t k0 = kbeg; k0 < kend; k0 += kKC) {
        __syncthreads();  // the previous stage is consumed
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int p = tid + 256 * l;
            Ps[p / kKC][p % kKC] = pv[l];
            if (QT)
                Qs[p / kKC][p % kKC] = qv[l];
            else
                Qs[p % TILE][p / TILE] = qv[l];
        }
        __syncthreads();
        if (k0 + kKC < kend) load(k0 + kKC);  // the next stage in flight
#pragma unroll
        for (int kk = 0; kk < kKC; kk += 4) {
            double a[MT], b[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) a[m] = Ps[ra + 16 * m][kk + lq];
#pragma unroll
            for (int n = 0; n < MT; ++n) b[n] = Qs[ca + 16 * n][kk + lq];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < MT; ++n)
                    acc.v[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], b[n], acc.v[m][n], 0,
                                                                       0, 0);
        }
    }
}

// Trailing update B[i][j] -= sum_{kbeg <= c < kend} B[i][c] B[j][c] for
// r0 <= j <= i < n and j < cend, on TILE x TILE tiles of the lower triangle
// (tile (ti, tj) starts at row r0 + TILE ti, column r0 + TILE tj).  Every
// entry's sum runs over c in the same order whatever the tile size.
template <int TILE>
__global__ __launch_bounds__(256) void syrk_update_kernel(double* __restrict__ B, int64_t n,
                                                          int64_t kbeg, int64_t kend, int64_t r0,
                                                          int64_t cend) {
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (tj > ti) return;  // lower tiles only; uniform over the block
    __shared__ __attribute__((aligned(16))) double Ps[TILE][kKP];
    __shared__ __attribute__((aligned(16))) double Qs[TILE][kKP];
    const int64_t ri0 = r0 + (int64_t)ti * TILE, rj0 = r0 + (int64_t)tj * TILE;
    auto ldp = [&](int r, int64_t k) -> double {
        return ri0 + r < n ? B[(ri0 + r) * n + k] : 0.0;
    };
    auto ldq = [&](int64_t k, int c) -> double {  // Q(k, c) = L[rj0 + c][k]
        return rj0 + c < cend ? B[(rj0 + c) * n + k] : 0.0;
    };
    TileAcc<TILE> acc;
    acc.zero();
    tile_product<TILE, true>(kbeg, kend, ldp, ldq, acc, Ps, Qs);
    acc.each([&](int r, int c, double v) {
        const int64_t i = ri0 + r, j = rj0 + c;
        if (i < n && j <= i && j < cend) B[i * n + j] -= v;
    });
}

// Inverse of every lower-triangular 64 x 64 diagonal block, in place
// (block x of the grid takes the block at 64 x): thread c forms column c by
// forward substitution.
__global__ __launch_bounds__(64) void trtri_diag_kernel(double* __restrict__ B, int64_t n) {
    __shared__ double L[kNB][kNB + 1];
    __shared__ double X[kNB][kNB + 1];
    const int64_t k0 = (int64_t)blockIdx.x * kNB;
    const int kb = (int)std::min<int64_t>(kNB, n - k0);
    const int c = threadIdx.x;
    for (int p = c; p < kb * kb; p += 64) {
        const int i = p / kb, j = p % kb;
        L[i][j] = j <= i ? B[(k0 + i) * n + k0 + j] : 0.0;
    }
    __syncthreads();
    if (c < kb) {
        X[c][c] = 1.0 / L[c][c];
        for (int i = c + 1; i < kb; ++i) {
            double s = 0.0;
            for (int m = c; m < i; ++m) s += L[i][m] * X[m][c];
            X[i][c] = -s / L[i][i];
        }
    }
    __syncthreads();
    for (int p = c; p < kb * kb; p += 64) {
        const int i = p / kb, j = p % kb;
        if (j <= i) B[(k0 + i) * n + k0 + j] = X[i][j];
    }
}

// One level of the recursive inverse, block size bs: pair z has
// A = [a0, a0 + bs), D = [a0 + bs, min(a0 + 2 bs, n)), a0 = 2 bs z; A^-1
// and D^-1 are already in place and B = C[D][A] is still the factor.
//   STEP 1: Tz[r][c] = sum_{k <= r} Dinv[r][k] B[k][c]  (T in scratch, pitch bs)
//   STEP 2: C[D][A][r][c] = -sum_{k >= c} Tz[r][k] Ainv[k][c]
template <int TILE, int STEP>
__global__ __launch_bounds__(256) void inv_level_kernel(double* __restrict__ B, int64_t n,
                                                        int64_t bs,
                                                        double* __restrict__ tmp) {
    __shared__ __attribute__((aligned(16))) double Ps[TILE][kKP];
    __shared__ __attribute__((aligned(16))) double Qs[TILE][kKP];
    const int64_t a0 = 2 * bs * (int64_t)blockIdx.z, d0 = a0 + bs;
    const int64_t dD = std::min<int64_t>(bs, n - d0);  // > 0: the host launches only such pairs
    const int64_t r0 = (int64_t)blockIdx.y * TILE, c0 = (int64_t)blockIdx.x * TILE;
    if (r0 >= dD) return;  // uniform
    double* T = tmp + (int64_t)blockIdx.z * bs * bs;
    TileAcc<TILE> acc;
    acc.zero();
    if (STEP == 1) {
        auto ldp = [&](int r, int64_t k) -> double {  // Dinv[r0 + r][k], k <= r
            const int64_t rr = r0 + r;
            return (rr < dD && k <= rr) ? B[(d0 + rr) * n + d0 + k] : 0.0;
        };
        auto ldq = [&](int64_t k, int c) -> double {  // B[d0 + k][a0 + c0 + c]
            return B[(d0 + k) * n + a0 + c0 + c];      // k < dD, c0 + c < bs
        };
        tile_product<TILE>(0, std::min<int64_t>(r0 + TILE, dD), ldp, ldq, acc, Ps, Qs);
    } else {
        auto ldp = [&](int r, int64_t k) -> double {  // T[r0 + r][k]
            const int64_t rr = r0 + r;
            return rr < dD ? T[rr * bs + k] : 0.0;
        };
        auto ldq = [&](int64_t k, int c) -> double {  // Ainv[k][c0 + c], k >= c0 + c
            return k >= c0 + c ? B[(a0 + k) * n + a0 + c0 + c] : 0.0;
        };
        tile_product<TILE>(c0, bs, ldp, ldq, acc, Ps, Qs);
    }
    acc.each([&](int r, int c, double v) {
        const int64_t rr = r0 + r, cc = c0 + c;
        if (rr >= dD) return;
        if (STEP == 1)
            T[rr * bs + cc] = v;
        else
            B[(d0 + rr) * n + a0 + cc] = -v;
    });
}

// U[i][j] = Cinv[n-1-i][n-1-j] for j >= i, 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const double* __restrict__ B, int64_t n,
                                                      float* __restrict__ U) {
    const int64_t i = blockIdx.y;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n;
         j += (int64_t)gridDim.x * 256)
        U[i * n + j] = j >= i ? (float)B[(n - 1 - i) * n + (n - 1 - j)] : 0.0f;
}

}  // namespace

// Scratch of the recursive inverse: per level, pairs x bs x bs doubles,
// at most about n^2 / 2.
static int64_t inv_scratch(int64_t n) {
    int64_t most = 0;
    for (int64_t bs = kNB; bs < n; bs *= 2) {
        const int64_t pairs = (n + 2 * bs - 1) / (2 * bs);
        most = std::max(most, pairs * bs * bs);
    }
    return most;
}

size_t gptq_factor_workspace(int64_t n) {
    // B (n x n f64) + the inverse's scratch + one f64 slot
    return (size_t)(n * n + inv_scratch(n) + 2) * sizeof(double);
}

hipError_t launch_gptq_factor(const float* H, int64_t n, double damp, float* U, int32_t* info,
                              void* workspace, hipStream_t s) {
    double* B = static_cast<double*>(workspace);
    double* tmp = B + n * n;
    double* add = tmp + inv_scratch(n);
    const unsigned rows = (unsigned)n;  // one grid row per matrix row
    const unsigned cols = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, s, H, n, damp, add, info);
    hipLaunchKernelGGL(reverse_kernel, dim3(cols, rows), dim3(256), 0, s, H, n, add, B);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Outer panels of kOuter columns, each factored in kNB-wide steps whose
    // updates stay inside the panel; then one rank-kOuter update of
    // everything right of and below it.  A strip of kNB columns takes
    // 64 x 64 tiles (128-wide ones would be half empty and twice as few).
    auto update = [&](int64_t kbeg, int64_t kend, int64_t r0, int64_t cend) {
        const int64_t rows = n - r0, cols = cend - r0;
        if (rows <= 0 || cols <= 0) return;
        if (cols <= kNB) {
            const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
            hipLaunchKernelGGL((syrk_update_kernel<64>), grid, dim3(256), 0, s, B, n, kbeg, kend,
                               r0, cend);
        } else {
            const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
            hipLaunchKernelGGL((syrk_update_kernel<128>), grid, dim3(256), 0, s, B, n, kbeg, kend,
                               r0, cend);
        }
    };
    for (int64_t K0 = 0; K0 < n; K0 += kOuter) {
        const int64_t K1 = std::min<int64_t>(K0 + kOuter, n);
        for (int64_t k0 = K0; k0 < K1; k0 += kNB) {
            const int kb = (int)std::min<int64_t>(kNB, n - k0);
            hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, s, B, n, k0, kb, info);
            const int64_t rest = n - k0 - kb;
            if (rest > 0) {  // kb == 64 here: only the last panel can be narrower
                hipLaunchKernelGGL(trsm_panel_kernel, dim3((unsigned)((rest + 15) / 16)),
                                   dim3(64), 0, s, B, n, k0);
                update(k0, k0 + kb, k0 + kb, K1);  // the rest of this outer panel
            }
        }
        update(K0, K1, K1, n);  // everything after it
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(trtri_diag_kernel, dim3((unsigned)((n + kNB - 1) / kNB)), dim3(64), 0, s,
                       B, n);
    for (int64_t bs = kNB; bs < n; bs *= 2) {
        // pairs whose D half is not empty
        const int64_t pairs = (n - bs + 2 * bs - 1) / (2 * bs);
        if (pairs > 65535) return hipErrorInvalidConfiguration;
        const int tile = bs >= 128 ? 128 : 64;
        const unsigned tiles = (unsigned)((bs + tile - 1) / tile);
        const dim3 grid(tiles, tiles, (unsigned)pairs);
        if (tile == 128) {
            hipLaunchKernelGGL((inv_level_kernel<128, 1>), grid, dim3(256), 0, s, B, n, bs, tmp);
            hipLaunchKernelGGL((inv_level_kernel<128, 2>), grid, dim3(256), 0, s, B, n, bs, tmp);
        } else {
            hipLaunchKernelGGL((inv_level_kernel<64, 1>), grid, dim3(256), 0, s, B, n, bs, tmp);
            hipLaunchKernelGGL((inv_level_kernel<64, 2>), grid, dim3(256), 0, s, B, n, bs, tmp);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(write_u_kernel, dim3(cols, rows), dim3(256), 0, s, B, n, U);
    return hipGetLastError();
}

}  // namespace qt
