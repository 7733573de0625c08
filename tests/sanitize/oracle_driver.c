/*
 * Runs every function of the CPU oracle (oracle/oracle.c, built together with
 * this file with AddressSanitizer and UndefinedBehaviorSanitizer) on small
 * inputs with short tail groups, and checks a few facts each result must
 * satisfy: codes in range, pack/unpack round trips, dequantize-then-multiply
 * equal to the f64 matvec, sampled matmul equal to the matvec, the f32
 * matvec near the f64 one, Hessian diagonal equal to the full Hessian's
 * diagonal, the GPTQ factor upper triangular with a positive diagonal.
 * Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "oracle.h"

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

/* xorshift draws in [-1, 1) */
static uint32_t rng_state = 12345u;
static float draw(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return (float)(rng_state >> 8) / 8388608.0f - 1.0f;
}

static void fill(float* a, int64_t n, float scale) {
    for (int64_t i = 0; i < n; ++i) a[i] = scale * draw();
}

static void run_shape(int64_t O, int64_t I) {
    const int64_t G = qto_groups(I);
    CHECK(G == (I + 63) / 64);
    float* W = malloc(sizeof(float) * O * I);
    float* d = malloc(sizeof(float) * I);
    float* x = malloc(sizeof(float) * I);
    float* scales = malloc(sizeof(float) * O * G);
    float* errs = malloc(sizeof(float) * O * G * 64);
    int8_t* codes = malloc(O * I);
    int8_t* back = malloc(O * I);
    uint8_t* gidx = malloc(O * G);
    uint8_t* packed = malloc(qto_packed_bytes(O, I));
    double* y = malloc(sizeof(double) * O);
    double* ay = malloc(sizeof(double) * O);
    double* What = malloc(sizeof(double) * O * I);
    float* yf = malloc(sizeof(float) * O);
    fill(W, O * I, 0.05f);
    for (int64_t i = 0; i < I; ++i) d[i] = 1.0f + draw();
    fill(x, I, 1.0f);

    /* grid search with importance, and plain absmax/4 */
    qto_quantize_g64(W, O, I, d, 64, 0.5f, 1.0f, scales, codes, gidx, errs);
    for (int64_t i = 0; i < O * I; ++i) CHECK(codes[i] >= -4 && codes[i] <= 3);
    for (int64_t i = 0; i < O * G; ++i) CHECK(gidx[i] < 64 && scales[i] >= 0.0f);
    qto_quantize_g64(W, O, I, NULL, 0, 0.5f, 1.0f, scales, codes, NULL, NULL);
    for (int64_t i = 0; i < O * I; ++i) CHECK(codes[i] >= -4 && codes[i] <= 3);

    /* pack / unpack round trip */
    qto_pack_i3(codes, O, I, packed);
    qto_unpack_i3(packed, O, I, back);
    for (int64_t i = 0; i < O * I; ++i) CHECK(back[i] == codes[i]);

    /* dequantize-then-multiply equals the f64 matvec (same f64 products) */
    qto_matvec_f64(packed, scales, O, I, x, y, ay);
    qto_dequant_f64(packed, scales, O, I, What);
    for (int64_t o = 0; o < O; ++o) {
        double s = 0.0;
        for (int64_t i = 0; i < I; ++i) s += What[o * I + i] * (double)x[i];
        CHECK(fabs(s - y[o]) <= 1e-9 * (ay[o] + 1e-30));
    }
    qto_matvec_f32(packed, scales, O, I, x, yf);
    for (int64_t o = 0; o < O; ++o) CHECK(fabs((double)yf[o] - y[o]) <= 1e-5 * (ay[o] + 1e-30));

    /* sampled matmul rows equal the matvec */
    {
        int64_t t_idx[3] = {0, 1, 1}, o_idx[3] = {0, O - 1, O / 2};
        float* X = malloc(sizeof(float) * 2 * I);
        for (int64_t i = 0; i < I; ++i) X[i] = x[i], X[I + i] = x[i];
        double ys[3], as[3];
        qto_matmul_f64_sampled(packed, scales, O, I, X, 2, 3, t_idx, o_idx, ys, as);
        for (int k = 0; k < 3; ++k) CHECK(ys[k] == y[o_idx[k]] && as[k] == ay[o_idx[k]]);
        free(X);
    }

    /* signed search */
    qto_quantize_g64_signed(W, O, I, d, 64, 32, 0.5f, 1.0f, scales, codes);
    for (int64_t i = 0; i < O * I; ++i) CHECK(codes[i] >= -4 && codes[i] <= 3);

    /* row-int reconstruction */
    qto_rowint_recon(W, O, I, 4, What);
    for (int64_t i = 0; i < O * I; ++i) CHECK(isfinite(What[i]));

    /* grouped int4 */
    {
        uint8_t* p4 = malloc(qto_packed_bytes_i4(O, I));
        qto_quantize_g64_i4(W, O, I, d, 64, 0.5f, 1.0f, scales, codes, gidx);
        for (int64_t i = 0; i < O * I; ++i) CHECK(codes[i] >= -8 && codes[i] <= 7);
        qto_pack_i4(codes, O, I, p4);
        qto_unpack_i4(p4, O, I, back);
        for (int64_t i = 0; i < O * I; ++i) CHECK(back[i] == codes[i]);
        qto_matvec_i4_f64(p4, scales, O, I, x, y, ay);
        for (int64_t o = 0; o < O; ++o) CHECK(isfinite(y[o]) && ay[o] >= fabs(y[o]));
        free(p4);
    }
    free(W); free(d); free(x); free(scales); free(errs); free(codes); free(back); free(gidx);
    free(packed); free(y); free(ay); free(What); free(yf);
}

static void run_hessian_and_gptq(int64_t T, int64_t O, int64_t I) {
    const int64_t G = qto_groups(I);
    float* X = malloc(sizeof(float) * T * I);
    double* dd = malloc(sizeof(double) * I);
    double* H = malloc(sizeof(double) * I * I);
    double* U = malloc(sizeof(double) * I * I);
    float* Hf = malloc(sizeof(float) * I * I);
    float* Uf = malloc(sizeof(float) * I * I);
    float* W = malloc(sizeof(float) * O * I);
    float* scales = malloc(sizeof(float) * O * G);
    int8_t* codes = malloc(O * I);
    double* wt = malloc(sizeof(double) * O * I);
    double* base = malloc(sizeof(double) * O * G);
    fill(X, T * I, 1.0f);
    fill(W, O * I, 0.05f);
    qto_hessian_diag(X, T, I, NULL, dd);
    qto_hessian_full(X, T, I, H);
    for (int64_t i = 0; i < I; ++i) CHECK(fabs(H[i * I + i] - dd[i]) <= 1e-12 * (dd[i] + 1e-30));
    for (int64_t i = 0; i < I; ++i)
        for (int64_t j = 0; j < I; ++j) CHECK(H[i * I + j] == H[j * I + i]);
    CHECK(qto_gptq_factor(H, I, 0.01, U) == 0);
    for (int64_t i = 0; i < I; ++i) {
        CHECK(U[i * I + i] > 0.0);
        for (int64_t j = 0; j < i; ++j) CHECK(U[i * I + j] == 0.0);
    }
    for (int64_t i = 0; i < I * I; ++i) Uf[i] = (float)U[i], Hf[i] = (float)H[i];
    qto_gptq_i3(W, O, I, Uf, 128, scales, codes);
    for (int64_t i = 0; i < O * I; ++i) CHECK(codes[i] >= -4 && codes[i] <= 3);
    qto_gptq_replay(W, O, I, Uf, scales, codes, wt, base);
    for (int64_t i = 0; i < O * I; ++i) CHECK(isfinite(wt[i]));
    {
        double num = 0.0, den = 0.0;
        qto_proxy_terms(W, O, I, codes, scales, Hf, &num, &den);
        CHECK(num >= 0.0 && den > 0.0);
    }
    free(X); free(dd); free(H); free(U); free(Hf); free(Uf); free(W); free(scales);
    free(codes); free(wt); free(base);
}

int main(void) {
    CHECK(qto_grid_factor(63, 64, 0.5f, 1.0f) == 1.0f);
    CHECK(qto_grid_factor(0, 64, 0.5f, 1.0f) == 0.5f);
    const int64_t shapes[][2] = {{3, 64}, {5, 130}, {4, 200}, {2, 1}, {7, 63}, {1, 259}};
    for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
        run_shape(shapes[s][0], shapes[s][1]);
    run_hessian_and_gptq(40, 6, 150);
    run_hessian_and_gptq(9, 3, 64);
    printf("%d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
