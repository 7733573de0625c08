// The GPTQ factor on the device: U = the upper Cholesky factor of A^-1,
// A = H + damp * mean(diag H) * I (the tt-stack issue page, pipeline table
// step 2: a Cholesky / inverse of H, there on the host with LAPACK, "blocked
// Cholesky on device later").
//
// With J the reversal, J A J = C C^T (C lower); then U = J C^-1 J is upper
// with U^T U = A^-1.  Everything runs in f64 on the vector ALUs (gfx950's
// f64 vector and matrix rates are the same), in 64-wide panels:
//   Cholesky, right-looking: factor the diagonal block in LDS, solve the
//   panel below it row by row, subtract the panel's outer product from the
//   trailing lower triangle;
//   inverse, from the last panel back: invert the diagonal block, then the
//   panel below it becomes -C^-1[rest, rest] C[rest, panel] Cinv[panel, panel]
//   (the trailing inverse is already in place; the product goes through a
//   scratch panel because it overwrites its own input).
// A non-positive pivot sets *info to its 1-based column (of the reversed
// matrix) and is replaced by 1 so that every later step stays finite.
#include <algorithm>

#include "qt_internal.h"

namespace qt {
namespace {

constexpr int kNB = 64;  // panel width

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

// Unblocked Cholesky of the kb x kb diagonal block at (k0, k0), in LDS.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ B, int64_t n,
                                                         int64_t k0, int kb,
                                                         int32_t* __restrict__ info) {
    __shared__ double T[kNB][kNB + 1];
    const int tid = threadIdx.x;
    for (int p = tid; p < kb * kb; p += 256) {
        const int i = p / kb, j = p % kb;
        T[i][j] = j <= i ? B[(k0 + i) * n + k0 + j] : 0.0;
    }
    __syncthreads();
    for (int c = 0; c < kb; ++c) {
        if (tid == 0) {
            double d = T[c][c];
            if (!(d > 0.0)) {
                if (*info == 0) *info = (int32_t)(k0 + c + 1);
                d = 1.0;
            }
            T[c][c] = sqrt(d);
        }
        __syncthreads();
        for (int i = c + 1 + tid; i < kb; i += 256) T[i][c] = T[i][c] / T[c][c];
        __syncthreads();
        const int m = kb - 1 - c;  // trailing size
        for (int p = tid; p < m * m; p += 256) {
            const int i = c + 1 + p / m, j = c + 1 + p % m;
            if (j <= i) T[i][j] -= T[i][c] * T[j][c];
        }
        __syncthreads();
    }
    for (int p = tid; p < kb * kb; p += 256) {
        const int i = p / kb, j = p % kb;
        if (j <= i) B[(k0 + i) * n + k0 + j] = T[i][j];
    }
}

// Rows below the diagonal block: x C_kk^T = b, one thread per row (64 values
// in registers, forward substitution over the columns).
__global__ __launch_bounds__(64) void trsm_panel_kernel(double* __restrict__ B, int64_t n,
                                                        int64_t k0) {
    __shared__ double L[kNB][kNB + 1];
    for (int p = threadIdx.x; p < kNB * kNB; p += 64) {
        const int i = p / kNB, j = p % kNB;
        L[i][j] = j <= i ? B[(k0 + i) * n + k0 + j] : 0.0;
    }
    __syncthreads();
    const int64_t r = k0 + kNB + (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (r >= n) return;
    double x[kNB];
    double* row = B + r * n + k0;
#pragma unroll
    for (int c = 0; c < kNB; ++c) x[c] = row[c];
#pragma unroll
    for (int c = 0; c < kNB; ++c) {
        double s = x[c];
#pragma unroll
        for (int m = 0; m < c; ++m) s -= x[m] * L[c][m];
        x[c] = s / L[c][c];
    }
#pragma unroll
    for (int c = 0; c < kNB; ++c) row[c] = x[c];
}

// 64 x 64 tile product helper: acc[a][b] += sum_c P[c][4ty+a] * Q[c][4tx+b]
// with P, Q in LDS as [c][row].
__device__ __forceinline__ void tile_fma(const double (*P)[kNB + 2], const double (*Q)[kNB + 2],
                                         int ty, int tx, double (&acc)[4][4]) {
#pragma unroll 4
    for (int c = 0; c < kNB; ++c) {
        double a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = P[c][4 * ty + u];
            b[u] = Q[c][4 * tx + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(a[u], b[v], acc[u][v]);
    }
}

// Trailing update B[i][j] -= sum_c B[i][k0+c] B[j][k0+c] for k0+64 <= j <= i.
__global__ __launch_bounds__(256) void syrk_update_kernel(double* __restrict__ B, int64_t n,
                                                          int64_t k0) {
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (tj > ti) return;  // lower tiles only; uniform over the block
    __shared__ double P[kNB][kNB + 2];
    __shared__ double Q[kNB][kNB + 2];
    const int64_t k1 = k0 + kNB;
    const int64_t ri0 = k1 + (int64_t)ti * kNB, rj0 = k1 + (int64_t)tj * kNB;
    const int tid = threadIdx.x;
    for (int p = tid; p < kNB * kNB; p += 256) {
        const int r = p / kNB, c = p % kNB;
        P[c][r] = ri0 + r < n ? B[(ri0 + r) * n + k0 + c] : 0.0;
        Q[c][r] = rj0 + r < n ? B[(rj0 + r) * n + k0 + c] : 0.0;
    }
    __syncthreads();
    const int ty = tid >> 4, tx = tid & 15;
    double acc[4][4] = {};
    tile_fma(P, Q, ty, tx, acc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = ri0 + 4 * ty + u;
        if (i >= n) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t j = rj0 + 4 * tx + v;
            if (j <= i) B[i * n + j] -= acc[u][v];
        }
    }
}

// Inverse of the lower-triangular diagonal block at (k0, k0), in place:
// thread c forms column c by forward substitution.
__global__ __launch_bounds__(64) void trtri_diag_kernel(double* __restrict__ B, int64_t n,
                                                        int64_t k0, int kb) {
    __shared__ double L[kNB][kNB + 1];
    __shared__ double X[kNB][kNB + 1];
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

// Panel below the diagonal block in the inverse: for the 64-row tile at r0,
// T = sum over 64-column tiles m0 in [k1, r0] of Cinv[r0.., m0..] C[m0.., k0..]
// (Cinv of the trailing part is final; its diagonal tile is lower triangular),
// then tmp[r0 - k1 ..] = -T Cinv[k0.., k0..].
__global__ __launch_bounds__(256) void trmm_panel_kernel(const double* __restrict__ B, int64_t n,
                                                         int64_t k0,
                                                         double* __restrict__ tmp) {
    __shared__ double P[kNB][kNB + 2];
    __shared__ double Q[kNB][kNB + 2];
    const int64_t k1 = k0 + kNB;
    const int64_t r0 = k1 + (int64_t)blockIdx.x * kNB;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    double acc[4][4] = {};
    for (int64_t m0 = k1; m0 <= r0; m0 += kNB) {
        __syncthreads();
        for (int p = tid; p < kNB * kNB; p += 256) {
            const int a = p / kNB, b = p % kNB;
            // P[c][r] = Cinv[r0 + r][m0 + c] (zero above the diagonal and past n)
            const int64_t r = r0 + a, m = m0 + b;
            P[b][a] = (r < n && m < n && m <= r) ? B[r * n + m] : 0.0;
            // Q[c][j] = C[m0 + c][k0 + j]
            Q[a][b] = (m0 + a < n) ? B[(m0 + a) * n + k0 + b] : 0.0;
        }
        __syncthreads();
        tile_fma(P, Q, ty, tx, acc);
    }
    // tmp tile = -T Cinv_kk: T to LDS as [row][c], then P[c][r] = T[r][c]
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) P[4 * tx + v][4 * ty + u] = acc[u][v];
    for (int p = tid; p < kNB * kNB; p += 256) {
        const int a = p / kNB, b = p % kNB;  // Q[c][j] = Cinv_kk[c][j]
        Q[a][b] = b <= a ? B[(k0 + a) * n + k0 + b] : 0.0;
    }
    __syncthreads();
    double out[4][4] = {};
    tile_fma(P, Q, ty, tx, out);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t r = r0 + 4 * ty + u;
        if (r >= n) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) tmp[(r - k1) * kNB + 4 * tx + v] = -out[u][v];
    }
}

__global__ __launch_bounds__(256) void copy_panel_kernel(double* __restrict__ B, int64_t n,
                                                         int64_t k0,
                                                         const double* __restrict__ tmp) {
    const int64_t k1 = k0 + kNB;
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = k1 + p / kNB;
    if (r >= n) return;
    B[r * n + k0 + p % kNB] = tmp[p];
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

size_t gptq_factor_workspace(int64_t n) {
    // B (n x n f64) + scratch panel (n x 64 f64) + one f64 slot
    return (size_t)(n * n + n * kNB + 2) * sizeof(double);
}

hipError_t launch_gptq_factor(const float* H, int64_t n, double damp, float* U, int32_t* info,
                              void* workspace, hipStream_t s) {
    double* B = static_cast<double*>(workspace);
    double* tmp = B + n * n;
    double* add = tmp + n * kNB;
    const unsigned rows = (unsigned)n;  // one grid row per matrix row
    const unsigned cols = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, s, H, n, damp, add, info);
    hipLaunchKernelGGL(reverse_kernel, dim3(cols, rows), dim3(256), 0, s, H, n, add, B);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int64_t k0 = 0; k0 < n; k0 += kNB) {
        const int kb = (int)std::min<int64_t>(kNB, n - k0);
        hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, s, B, n, k0, kb, info);
        const int64_t rest = n - k0 - kb;
        if (rest > 0) {  // kb == 64 here: only the last panel can be narrower
            hipLaunchKernelGGL(trsm_panel_kernel, dim3((unsigned)((rest + 63) / 64)), dim3(64), 0,
                               s, B, n, k0);
            const unsigned mt = (unsigned)((rest + kNB - 1) / kNB);
            hipLaunchKernelGGL(syrk_update_kernel, dim3(mt, mt), dim3(256), 0, s, B, n, k0);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t last = (n - 1) / kNB * kNB;
    for (int64_t k0 = last; k0 >= 0; k0 -= kNB) {
        const int kb = (int)std::min<int64_t>(kNB, n - k0);
        hipLaunchKernelGGL(trtri_diag_kernel, dim3(1), dim3(64), 0, s, B, n, k0, kb);
        const int64_t rest = n - k0 - kb;
        if (rest > 0) {
            const unsigned mt = (unsigned)((rest + kNB - 1) / kNB);
            hipLaunchKernelGGL(trmm_panel_kernel, dim3(mt), dim3(256), 0, s, B, n, k0, tmp);
            hipLaunchKernelGGL(copy_panel_kernel, dim3((unsigned)((rest * kNB + 255) / 256)),
                               dim3(256), 0, s, B, n, k0, tmp);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(write_u_kernel, dim3(cols, rows), dim3(256), 0, s, B, n, U);
    return hipGetLastError();
}

}  // namespace qt
