/*
 * int3-g64 CPU oracle -- TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Plain scalar C.  Build: gcc -O2 -ffp-contract=off -fno-fast-math.  Every f32
 * expression below is written one operation per statement so that the value
 * of each rounding step is the one the text describes.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#define GROUP 64

int64_t qto_groups(int64_t I) { return (I + GROUP - 1) / GROUP; }

/* Pull request page, "Design": 24 bytes per row per 64-input group. */
int64_t qto_packed_bytes(int64_t O, int64_t I) { return O * qto_groups(I) * 24; }

/* NeUQI page, first paragraph: a grid search over candidate scales.  The grid
 * is read as n equally spaced points of the closed interval [lo, hi]
 * (numpy.linspace semantics: start + k*step, the last point set to stop). */
float qto_grid_factor(int k, int n, float lo, float hi) {
    if (k == n - 1) return hi;
    double step = ((double)hi - (double)lo) / (double)(n - 1);
    double f = (double)lo + (double)k * step;
    return (float)f;
}

/* Round-to-nearest-even of the correctly rounded f32 quotient w/s, clamped
 * to the code range [cmin, cmax]: [-4, 3] for int3-g64 (pull request page,
 * "Design", Layout), [-8, 7] for grouped int4. */
static int code_in(float w, float s, float cmin, float cmax) {
    if (s == 0.0f) return 0;
    float q = w / s;
    float r = rintf(q); /* default rounding mode: to nearest, ties to even */
    if (r < cmin) r = cmin;
    if (r > cmax) r = cmax;
    return (int)r;
}

static int code_for(float w, float s) { return code_in(w, s, -4.0f, 3.0f); }

/* Weighted squared reconstruction error of one group at scale s, the search
 * objective: every slot's error d*(w - s*q)^2 with each operation a rounded
 * f32 operation (padding slots of a short tail group contribute zero), then
 * the pairwise halving sum a[j] += a[j+m], m = 32, 16, ..., 1. */
static float group_error_in(const float* w, int n, const float* dg, float s, float cmin,
                            float cmax) {
    float a[GROUP];
    for (int j = 0; j < GROUP; ++j) {
        if (j < n) {
            const int q = code_in(w[j], s, cmin, cmax);
            const float t = s * (float)q;
            const float r = w[j] - t;
            const float r2 = r * r;
            a[j] = dg ? dg[j] * r2 : r2;
        } else {
            a[j] = 0.0f;
        }
    }
    for (int m = GROUP / 2; m >= 1; m /= 2)
        for (int j = 0; j < m; ++j) a[j] = a[j] + a[j + m];
    return a[0];
}

static float group_error(const float* w, int n, const float* dg, float s) {
    return group_error_in(w, n, dg, s, -4.0f, 3.0f);
}

/* base scale: absmax over the group's real values, times 1/4 (a 3-bit
 * symmetric quantizer: 2^(3-1) = 4 levels per side) */
static float group_base(const float* w, int n) {
    float amax = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(w[j]);
        if (a > amax) amax = a;
    }
    return amax * 0.25f;
}

void qto_quantize_g64(const float* W, int64_t O, int64_t I, const float* d,
                      int n_grid, float lo, float hi, float* scales,
                      int8_t* codes, uint8_t* grid_idx, float* errs) {
    const int64_t G = qto_groups(I);
    const int ncand = n_grid == 0 ? 1 : n_grid;
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t c0 = g * GROUP;
            const int n = (int)((I - c0) < GROUP ? (I - c0) : GROUP);
            const float* w = W + o * I + c0;
            const float base = group_base(w, n);

            int best_k = 0;
            float best_e = 0.0f;
            for (int k = 0; k < ncand; ++k) {
                const float f = n_grid == 0 ? 1.0f : qto_grid_factor(k, n_grid, lo, hi);
                const float s = base * f;
                const float e = group_error(w, n, d ? d + c0 : NULL, s);
                if (errs) errs[(o * G + g) * ncand + k] = e;
                if (k == 0 || e < best_e) { /* lowest k wins ties */
                    best_e = e;
                    best_k = k;
                }
            }
            const float f = n_grid == 0 ? 1.0f : qto_grid_factor(best_k, n_grid, lo, hi);
            const float s = base * f;
            scales[o * G + g] = s;
            if (grid_idx) grid_idx[o * G + g] = (uint8_t)best_k;
            for (int j = 0; j < n; ++j) codes[o * I + c0 + j] = (int8_t)code_for(w[j], s);
        }
    }
}

/* NeUQI page, first paragraph and results notes: symmetric layers use a
 * two-stage signed scale search, 64 then 32 points by default ("64/32").
 * Reading of the stages (the pages give no formula):
 *   stage 1: the n1-point grid f_k of [lo, hi] times base, each factor with
 *            both signs, candidate order k ascending, + before - (a negative
 *            scale lets the largest |w| take the -4 level);
 *   stage 2: n2 points of [f_{k-1}, f_{k+1}] around the stage-1 winner k
 *            (clipped to the grid ends), same linspace rule, with the
 *            winner's sign;
 *   the final choice is the strict minimum over [stage-1 winner, stage-2
 *   points in order], so ties keep the earlier candidate and the result is
 *   never worse than stage 1.  n2 == 0: stage 1 only. */
void qto_quantize_g64_signed(const float* W, int64_t O, int64_t I, const float* d, int n1,
                             int n2, float lo, float hi, float* scales, int8_t* codes) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t c0 = g * GROUP;
            const int n = (int)((I - c0) < GROUP ? (I - c0) : GROUP);
            const float* w = W + o * I + c0;
            const float* dg = d ? d + c0 : NULL;
            const float base = group_base(w, n);

            int best_k = 0, best_neg = 0, first = 1;
            float best_e = 0.0f;
            for (int k = 0; k < n1; ++k) {
                for (int neg = 0; neg < 2; ++neg) {
                    const float mag = base * qto_grid_factor(k, n1, lo, hi);
                    const float s = neg ? -mag : mag;
                    const float e = group_error(w, n, dg, s);
                    if (first || e < best_e) {
                        best_e = e;
                        best_k = k;
                        best_neg = neg;
                        first = 0;
                    }
                }
            }
            const float mag1 = base * qto_grid_factor(best_k, n1, lo, hi);
            float best_s = best_neg ? -mag1 : mag1;
            if (n2 > 0) {
                const float a = qto_grid_factor(best_k > 0 ? best_k - 1 : 0, n1, lo, hi);
                const float b = qto_grid_factor(best_k < n1 - 1 ? best_k + 1 : n1 - 1, n1, lo, hi);
                for (int j = 0; j < n2; ++j) {
                    const float mag = base * qto_grid_factor(j, n2, a, b);
                    const float s = best_neg ? -mag : mag;
                    const float e = group_error(w, n, dg, s);
                    if (e < best_e) {
                        best_e = e;
                        best_s = s;
                    }
                }
            }
            scales[o * G + g] = best_s;
            for (int j = 0; j < n; ++j) codes[o * I + c0 + j] = (int8_t)code_for(w[j], best_s);
        }
    }
}

/* Pull request page, "Design", Layout: low plane first (2 bits per value, 16
 * bytes), then the high plane (1 bit per value, 8 bytes), of u = v + 4.
 * Reading of the bit order (the pages print no byte): value 4b+i sits in bits
 * 2i..2i+1 of low byte b, value 8c+i in bit i of high byte c.  Padding slots of
 * a short tail group hold v = 0. */
void qto_pack_i3(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t c0 = g * GROUP;
            const int n = (int)((I - c0) < GROUP ? (I - c0) : GROUP);
            uint8_t* p = packed + (o * G + g) * 24;
            for (int b = 0; b < 24; ++b) p[b] = 0;
            for (int j = 0; j < GROUP; ++j) {
                const int v = j < n ? codes[o * I + c0 + j] : 0;
                const int u = v + 4;
                p[j / 4] |= (uint8_t)((u & 3) << (2 * (j % 4)));
                p[16 + j / 8] |= (uint8_t)(((u >> 2) & 1) << (j % 8));
            }
        }
    }
}

/* stored code of slot j of one 24-byte group, as v = u - 4 */
static int code_at(const uint8_t* p, int j) {
    const int lo = (p[j / 4] >> (2 * (j % 4))) & 3;
    const int hi = (p[16 + j / 8] >> (j % 8)) & 1;
    return (lo | (hi << 2)) - 4;
}

void qto_unpack_i3(const uint8_t* packed, int64_t O, int64_t I, int8_t* codes) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i)
            codes[o * I + i] = (int8_t)code_at(packed + (o * G + i / GROUP) * 24, (int)(i % GROUP));
}

void qto_dequant_f64(const uint8_t* packed, const float* scales, int64_t O,
                     int64_t I, double* What) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i) {
            const int64_t g = i / GROUP;
            const int v = code_at(packed + (o * G + g) * 24, (int)(i % GROUP));
            What[o * I + i] = (double)scales[o * G + g] * (double)v;
        }
}

/* fp64 dequantize-then-multiply (test method of the pull request page,
 * "Tests": the kernel against dequant-matmul). */
void qto_matvec_f64(const uint8_t* packed, const float* scales, int64_t O,
                    int64_t I, const float* x, double* y, double* absy) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o) {
        double acc = 0.0, aacc = 0.0;
        for (int64_t i = 0; i < I; ++i) {
            const int64_t g = i / GROUP;
            const int v = code_at(packed + (o * G + g) * 24, (int)(i % GROUP));
            const double w = (double)scales[o * G + g] * (double)v;
            const double p = w * (double)x[i];
            acc += p;
            aacc += fabs(p);
        }
        y[o] = acc;
        if (absy) absy[o] = aacc;
    }
}

void qto_matmul_f64_sampled(const uint8_t* packed, const float* scales,
                            int64_t O, int64_t I, const float* X, int64_t B,
                            int64_t n, const int64_t* t_idx,
                            const int64_t* o_idx, double* y, double* absy) {
    const int64_t G = qto_groups(I);
    (void)B;
    (void)O;
    for (int64_t k = 0; k < n; ++k) {
        const int64_t t = t_idx[k], o = o_idx[k];
        double acc = 0.0, aacc = 0.0;
        for (int64_t i = 0; i < I; ++i) {
            const int64_t g = i / GROUP;
            const int v = code_at(packed + (o * G + g) * 24, (int)(i % GROUP));
            const double w = (double)scales[o * G + g] * (double)v;
            const double p = w * (double)X[t * I + i];
            acc += p;
            aacc += fabs(p);
        }
        y[k] = acc;
        if (absy) absy[k] = aacc;
    }
}

/* Pull request page, "Design", Kernel bullet: exact-f32 path with per-group
 * scale accumulation. */
void qto_matvec_f32(const uint8_t* packed, const float* scales, int64_t O,
                    int64_t I, const float* x, float* y) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o) {
        float yo = 0.0f;
        for (int64_t g = 0; g < G; ++g) {
            const int64_t c0 = g * GROUP;
            const int n = (int)((I - c0) < GROUP ? (I - c0) : GROUP);
            const uint8_t* p = packed + (o * G + g) * 24;
            float acc = 0.0f;
            for (int j = 0; j < n; ++j) {
                const float prod = (float)code_at(p, j) * x[c0 + j];
                acc = acc + prod;
            }
            const float part = scales[o * G + g] * acc;
            yo = yo + part;
        }
        y[o] = yo;
    }
}

/* tt-stack page, pipeline table step 1: H = sum_t X^T X; its diagonal is the
 * per-column sum of squares over tokens.  Accumulated in double. */
void qto_hessian_diag(const float* X, int64_t T, int64_t I,
                      const double* d_in, double* d_out) {
    for (int64_t j = 0; j < I; ++j) d_out[j] = d_in ? d_in[j] : 0.0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < I; ++j) {
            const double v = (double)X[t * I + j];
            d_out[j] += v * v;
        }
}

/* Per-row b-bit absmax RTN (the shipped per-row int4 format that the pull
 * request page compares against). */
void qto_rowint_recon(const float* W, int64_t O, int64_t I, int bits,
                      double* recon) {
    const int half = 1 << (bits - 1);
    for (int64_t o = 0; o < O; ++o) {
        const float* w = W + o * I;
        float amax = 0.0f;
        for (int64_t i = 0; i < I; ++i) {
            float a = fabsf(w[i]);
            if (a > amax) amax = a;
        }
        const float s = amax / (float)half;
        for (int64_t i = 0; i < I; ++i) {
            float q = 0.0f;
            if (s != 0.0f) {
                float qq = w[i] / s;
                q = rintf(qq);
                if (q < (float)-half) q = (float)-half;
                if (q > (float)(half - 1)) q = (float)(half - 1);
            }
            recon[o * I + i] = (double)s * (double)q;
        }
    }
}


/* ------------------------------------------------------------------ grouped int4
 * The pull request page names group-scaled int4 (the format number it took,
 * and grouped int4 at gs = 64 carrying the same O*ceil(I/64) scale count); it
 * prints no layout.  Readings: a 4-bit symmetric absmax quantizer per
 * 64-input group (base = absmax * 2^-(4-1) = absmax/8, codes in [-8, 7]), the
 * same objective, grid and tie rule as int3-g64; storage per group 32 bytes of
 * u = v + 8, code j in the low nibble of byte j/2 for even j and in the high
 * nibble for odd j; one f32 scale per group in its own tensor; short tail
 * groups padded with v = 0 (u = 8). */
int64_t qto_packed_bytes_i4(int64_t O, int64_t I) { return O * qto_groups(I) * 32; }

void qto_quantize_g64_i4(const float* W, int64_t O, int64_t I, const float* d, int n_grid,
                         float lo, float hi, float* scales, int8_t* codes, uint8_t* grid_idx) {
    const int64_t G = qto_groups(I);
    const int ncand = n_grid == 0 ? 1 : n_grid;
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t c0 = g * GROUP;
            const int n = (int)((I - c0) < GROUP ? (I - c0) : GROUP);
            const float* w = W + o * I + c0;
            float amax = 0.0f;
            for (int j = 0; j < n; ++j) {
                float a = fabsf(w[j]);
                if (a > amax) amax = a;
            }
            const float base = amax * 0.125f;
            int best_k = 0;
            float best_e = 0.0f;
            for (int k = 0; k < ncand; ++k) {
                const float f = n_grid == 0 ? 1.0f : qto_grid_factor(k, n_grid, lo, hi);
                const float s = base * f;
                const float e = group_error_in(w, n, d ? d + c0 : NULL, s, -8.0f, 7.0f);
                if (k == 0 || e < best_e) {
                    best_e = e;
                    best_k = k;
                }
            }
            const float f = n_grid == 0 ? 1.0f : qto_grid_factor(best_k, n_grid, lo, hi);
            const float s = base * f;
            scales[o * G + g] = s;
            if (grid_idx) grid_idx[o * G + g] = (uint8_t)best_k;
            for (int j = 0; j < n; ++j)
                codes[o * I + c0 + j] = (int8_t)code_in(w[j], s, -8.0f, 7.0f);
        }
    }
}

void qto_pack_i4(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t c0 = g * GROUP;
            const int n = (int)((I - c0) < GROUP ? (I - c0) : GROUP);
            uint8_t* p = packed + (o * G + g) * 32;
            for (int b = 0; b < 32; ++b) p[b] = 0;
            for (int j = 0; j < GROUP; ++j) {
                const int v = j < n ? codes[o * I + c0 + j] : 0;
                const int u = v + 8;
                p[j / 2] |= (uint8_t)((u & 15) << (4 * (j % 2)));
            }
        }
    }
}

static int code_at_i4(const uint8_t* p, int j) {
    return (int)((p[j / 2] >> (4 * (j % 2))) & 15) - 8;
}

void qto_unpack_i4(const uint8_t* packed, int64_t O, int64_t I, int8_t* codes) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i)
            codes[o * I + i] =
                (int8_t)code_at_i4(packed + (o * G + i / GROUP) * 32, (int)(i % GROUP));
}

void qto_matvec_i4_f64(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                       const float* x, double* y, double* absy) {
    const int64_t G = qto_groups(I);
    for (int64_t o = 0; o < O; ++o) {
        double acc = 0.0, aacc = 0.0;
        for (int64_t i = 0; i < I; ++i) {
            const int64_t g = i / GROUP;
            const int v = code_at_i4(packed + (o * G + g) * 32, (int)(i % GROUP));
            const double w = (double)scales[o * G + g] * (double)v;
            const double p = w * (double)x[i];
            acc += p;
            aacc += fabs(p);
        }
        y[o] = acc;
        if (absy) absy[o] = aacc;
    }
}


/* ------------------------------------------------------------------ GPTQ / LDLQ
 * tt-stack issue page, pipeline table: step 1 accumulates the full
 * H = sum over tokens of X^T X per linear input; step 2 factors H (Cholesky /
 * inverse, host LAPACK in f32/f64 there); step 3 is the GPTQ/LDLQ column sweep:
 * serial rounding inside 128-column blocks, then the matmul
 * W[:, rest] -= E Hinv[blk, rest] carrying each block's scaled rounding errors
 * E to the later columns.  The "Risks" paragraph gates on the proxy error
 * tr(E H E^T) / tr(W H W^T).  The page names the algorithm and prints none of
 * its formulas.  Readings, each stated where it applies:
 *   - damping: A = H + damp * mean(diag H) * I;
 *   - Hinv is the upper Cholesky factor U of A^-1 (U^T U = A^-1), the GPTQ
 *     form of the sweep: for column i, err = (w_i - s q_i) / U[i][i] and every
 *     later column j takes w_j -= err U[i][j];
 *   - Q is the int3-g64 rounder with the group scale fixed when the sweep
 *     reaches the group's first column: absmax/4 of the group's current
 *     (already updated) values;
 *   - precision: the factorization in f64; the sweep in f32 as the page's host
 *     propagator, every in-block update one fused multiply-add in column
 *     order; the propagation of a finished block summed in f64 and applied
 *     with one f32 rounding. */
void qto_hessian_full(const float* X, int64_t T, int64_t I, double* H) {
    for (int64_t i = 0; i < I; ++i)
        for (int64_t j = 0; j < I; ++j) H[i * I + j] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const float* x = X + t * I;
        for (int64_t i = 0; i < I; ++i) {
            const double xi = (double)x[i];
            for (int64_t j = 0; j < I; ++j) H[i * I + j] += xi * (double)x[j];
        }
    }
}

/* U = the upper Cholesky factor of A^-1, A = H + damp * mean(diag H) * I.
 * With J the reversal, J A J = C C^T (textbook Cholesky, C lower); then
 * A = V V^T for the upper V = J C J, A^-1 = (V^-1)^T V^-1, and U = V^-1 =
 * J C^-1 J (upper, positive diagonal: the Cholesky factor).  C^-1 comes from
 * forward substitution against the identity.  U is written as a full n x n
 * matrix with zeros below the diagonal.  Returns 0, or -1 when A is not
 * positive definite. */
int qto_gptq_factor(const double* H, int64_t n, double damp, double* U) {
    double mean = 0.0;
    for (int64_t i = 0; i < n; ++i) mean += H[i * n + i];
    mean /= (double)n;
    const double add = damp * mean;
    double* C = (double*)malloc((size_t)(n * n) * sizeof(double));
    if (!C) return -1;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double a = H[(n - 1 - i) * n + (n - 1 - j)];
            if (i == j) a += add;
            C[i * n + j] = a;
        }
    for (int64_t j = 0; j < n; ++j) {
        double s = C[j * n + j];
        for (int64_t k = 0; k < j; ++k) s -= C[j * n + k] * C[j * n + k];
        if (!(s > 0.0)) {
            free(C);
            return -1;
        }
        const double cjj = sqrt(s);
        C[j * n + j] = cjj;
        for (int64_t i = j + 1; i < n; ++i) {
            double t = C[i * n + j];
            for (int64_t k = 0; k < j; ++k) t -= C[i * n + k] * C[j * n + k];
            C[i * n + j] = t / cjj;
        }
    }
    /* Ci = C^-1, column c: C x = e_c by forward substitution (x_i = 0 for
     * i < c); then U[i][j] = Ci[n-1-i][n-1-j]. */
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j) U[i * n + j] = 0.0;
    double* x = (double*)malloc((size_t)n * sizeof(double));
    if (!x) {
        free(C);
        return -1;
    }
    for (int64_t c = 0; c < n; ++c) {
        for (int64_t i = c; i < n; ++i) {
            double t = (i == c) ? 1.0 : 0.0;
            for (int64_t k = c; k < i; ++k) t -= C[i * n + k] * x[k];
            x[i] = t / C[i * n + i];
        }
        for (int64_t i = c; i < n; ++i) U[(n - 1 - i) * n + (n - 1 - c)] = x[i];
    }
    free(x);
    free(C);
    return 0;
}

/* The GPTQ sweep with the int3-g64 rounder, one row at a time (rows are
 * independent): w holds the row's current values. */
void qto_gptq_i3(const float* W, int64_t O, int64_t I, const float* U, int block,
                 float* scales, int8_t* codes) {
    const int64_t G = qto_groups(I);
    float* w = (float*)malloc((size_t)I * sizeof(float));
    float* err = (float*)malloc((size_t)I * sizeof(float));
    if (!w || !err) {
        free(w);
        free(err);
        return;
    }
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t j = 0; j < I; ++j) w[j] = W[o * I + j];
        for (int64_t b0 = 0; b0 < I; b0 += block) {
            const int64_t b1 = (b0 + block < I) ? b0 + block : I;
            float s = 0.0f;
            for (int64_t i = b0; i < b1; ++i) {
                if (i % GROUP == 0) { /* group start: the scale of the current values */
                    const int64_t n = (I - i < GROUP) ? I - i : GROUP;
                    float amax = 0.0f;
                    for (int64_t m = 0; m < n; ++m) {
                        const float a = fabsf(w[i + m]);
                        if (a > amax) amax = a;
                    }
                    s = amax * 0.25f;
                    scales[o * G + i / GROUP] = s;
                }
                const int q = code_for(w[i], s);
                codes[o * I + i] = (int8_t)q;
                const float t = s * (float)q;
                const float r = w[i] - t;
                err[i] = r / U[i * I + i];
                for (int64_t j = i + 1; j < b1; ++j) w[j] = fmaf(-err[i], U[i * I + j], w[j]);
            }
            /* the finished block's errors reach every later column */
            for (int64_t j = b1; j < I; ++j) {
                double acc = 0.0;
                for (int64_t k = b0; k < b1; ++k) acc += (double)err[k] * (double)U[k * I + j];
                w[j] = (float)((double)w[j] - acc);
            }
        }
    }
    free(w);
    free(err);
}

/* The same sweep in f64, unblocked, along given codes and scales: wt[o][i]
 * receives the value of column i when it is rounded, base[o][g] the
 * absmax/4 of the group's values when the sweep reaches its first column.  A
 * sweep that followed the algorithm chose codes that round wt/s (up to the
 * rounding of its own arithmetic) and scales equal to base. */
void qto_gptq_replay(const float* W, int64_t O, int64_t I, const float* U,
                     const float* scales, const int8_t* codes, double* wt_out,
                     double* base_out) {
    const int64_t G = qto_groups(I);
    double* w = (double*)malloc((size_t)I * sizeof(double));
    if (!w) return;
    for (int64_t o = 0; o < O; ++o) {
        for (int64_t j = 0; j < I; ++j) w[j] = (double)W[o * I + j];
        for (int64_t i = 0; i < I; ++i) {
            if (i % GROUP == 0) {
                const int64_t n = (I - i < GROUP) ? I - i : GROUP;
                double amax = 0.0;
                for (int64_t m = 0; m < n; ++m) {
                    const double a = fabs(w[i + m]);
                    if (a > amax) amax = a;
                }
                base_out[o * G + i / GROUP] = amax * 0.25;
            }
            wt_out[o * I + i] = w[i];
            const double e = (w[i] - (double)scales[o * G + i / GROUP] * (double)codes[o * I + i]) /
                             (double)U[i * I + i];
            for (int64_t j = i + 1; j < I; ++j) w[j] -= e * (double)U[i * I + j];
        }
    }
    free(w);
}

/* Proxy terms of the gate: num = sum_o e_o H e_o^T with e = W - s*v (the
 * dequantized codes), den = sum_o w_o H w_o^T, in f64. */
void qto_proxy_terms(const float* W, int64_t O, int64_t I, const int8_t* codes,
                     const float* scales, const float* H, double* num, double* den) {
    const int64_t G = qto_groups(I);
    double* e = (double*)malloc((size_t)I * sizeof(double));
    if (!e) return;
    double sn = 0.0, sd = 0.0;
    for (int64_t o = 0; o < O; ++o) {
        const float* w = W + o * I;
        for (int64_t i = 0; i < I; ++i)
            e[i] = (double)w[i] - (double)scales[o * G + i / GROUP] * (double)codes[o * I + i];
        for (int64_t i = 0; i < I; ++i) {
            double hn = 0.0, hd = 0.0;
            for (int64_t j = 0; j < I; ++j) {
                hn += (double)H[i * I + j] * e[j];
                hd += (double)H[i * I + j] * (double)w[j];
            }
            sn += e[i] * hn;
            sd += (double)w[i] * hd;
        }
    }
    *num = sn;
    *den = sd;
    free(e);
}
