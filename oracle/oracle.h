/*
 * int3-g64 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded scalar C that states what the int3-g64 hot path
 * computes.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product library never does, and the two share
 * no source, header, table or helper.
 *
 * Sources (all on the pages this project is built from):
 *   - "int3-g64 (fmt=5)" pull request page, section "Design", Layout bullet:
 *     24 bytes per row per 64-input group = 16 B low plane (2 bits/value) +
 *     8 B high plane (1 bit/value); values in [-4,3] stored as v+4; one f32
 *     scale per group in a separate tensor.
 *   - same page, "Design", Kernel bullet: an exact-f32 matmul with per-group
 *     scale accumulation (matmul_i3).
 *   - same page, "Why this format" item 1: the group quantizer mirrors a
 *     3-bit, group-64 absmax quantizer; the outlier-row property
 *     (int3-g64 reconstruction RMS below per-row int4).
 *   - NeUQI accuracy page, first paragraph: a grid search over scales weighted
 *     by the activation importance.
 *   - tt-stack issue page, pipeline table step 1: H = sum over tokens of X^T X
 *     per linear input, accumulated in fp32 (the diagonal is used here).
 *
 * Conventions: row-major, G = ceil(I/64) groups per row, group g of a row
 * covers columns [64g, min(64g+64, I)).  All pointers are host pointers owned
 * by the caller.  Inputs must be finite.  Floating point follows IEEE-754
 * binary32/binary64 with round-to-nearest-even; the library is compiled
 * without contraction or fast-math so every f32 operation written is one
 * rounded operation.
 *
 * Parity status: every function here is pinned by the CPU tests (worked
 * byte examples, exhaustive round trips, brute-force search optimality, closed
 * forms and library routines); the low/high-plane bit order is a reading of
 * the pages, which print no packed byte (see the pack function).
 */
#ifndef QT_ORACLE_H
#define QT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int64_t qto_groups(int64_t I);
int64_t qto_packed_bytes(int64_t O, int64_t I);

/* Candidate factor f_k of an n-point closed grid on [lo, hi] (n >= 2),
 * computed in double and rounded once to float. */
float qto_grid_factor(int k, int n, float lo, float hi);

/* Group scale search and code emission.
 * n_grid == 0: one candidate, the plain absmax/4 scale.
 * n_grid in 2..256: candidates base*f_k, k = 0..n_grid-1.
 * d: importance per input column (I floats) or NULL (all ones).
 * Outputs: scales[O*G], codes[O*I] (values in [-4,3]), grid_idx[O*G] or NULL,
 * errs[O*G*max(n_grid,1)] or NULL (the f32 objective of every candidate). */
void qto_quantize_g64(const float* W, int64_t O, int64_t I, const float* d,
                      int n_grid, float lo, float hi, float* scales,
                      int8_t* codes, uint8_t* grid_idx, float* errs);

/* Two-stage signed scale search (NeUQI page): stage 1 over the n1-point grid
 * of [lo, hi] with both signs, stage 2 over n2 points between the stage-1
 * winner's neighbours with its sign (n2 == 0: stage 1 only).  Same objective,
 * rounding and tie rule as qto_quantize_g64; scales may be negative. */
void qto_quantize_g64_signed(const float* W, int64_t O, int64_t I, const float* d, int n1,
                             int n2, float lo, float hi, float* scales, int8_t* codes);

/* Bit-plane packer / unpacker (codes in [-4,3]; packed O*G*24 bytes). */
void qto_pack_i3(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed);
void qto_unpack_i3(const uint8_t* packed, int64_t O, int64_t I, int8_t* codes);

/* y[o] = sum_i (double)s[o,g(i)]*(double)v[o,i] * (double)x[i] in double
 * (fp64 dequantize-then-multiply); absy[o] = sum_i |w_hat[o,i]*x[i]|. */
void qto_matvec_f64(const uint8_t* packed, const float* scales, int64_t O,
                    int64_t I, const float* x, double* y, double* absy);

/* Y[t,o] for a list of (t, o) samples of Y = X * W_hat^T, X[B x I] f32
 * (bf16 inputs are passed widened to f32, which is exact). */
void qto_matmul_f64_sampled(const uint8_t* packed, const float* scales,
                            int64_t O, int64_t I, const float* X, int64_t B,
                            int64_t n, const int64_t* t_idx,
                            const int64_t* o_idx, double* y, double* absy);

/* The exact-f32 per-group path: per group an f32 sequential sum of v*x,
 * times the group scale, then an f32 sequential sum over groups. */
void qto_matvec_f32(const uint8_t* packed, const float* scales, int64_t O,
                    int64_t I, const float* x, float* y);

/* d_out[j] = d_in[j] (or 0 if d_in is NULL) + sum_t (double)X[t,j]^2. */
void qto_hessian_diag(const float* X, int64_t T, int64_t I,
                      const double* d_in, double* d_out);

/* Per-row symmetric b-bit RTN reconstruction: s = absmax(row) / 2^(b-1),
 * q = clamp(rint(w/s), -2^(b-1), 2^(b-1)-1), recon = (double)s*q. */
void qto_rowint_recon(const float* W, int64_t O, int64_t I, int bits,
                      double* recon);

/* int3-g64 reconstruction What[o,i] = (double)s[o,g(i)] * v[o,i] (exact). */
void qto_dequant_f64(const uint8_t* packed, const float* scales, int64_t O,
                     int64_t I, double* What);

/* Grouped int4 (the pull request page's group-scaled int4; layout read as
 * 32 bytes of u = v + 8 per 64-input group, low nibble first, v in [-8, 7],
 * base = absmax/8, search and objective as int3-g64). */
int64_t qto_packed_bytes_i4(int64_t O, int64_t I);
void qto_quantize_g64_i4(const float* W, int64_t O, int64_t I, const float* d, int n_grid,
                         float lo, float hi, float* scales, int8_t* codes, uint8_t* grid_idx);
void qto_pack_i4(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed);
void qto_unpack_i4(const uint8_t* packed, int64_t O, int64_t I, int8_t* codes);
void qto_matvec_i4_f64(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                       const float* x, double* y, double* absy);

/* GPTQ / LDLQ (tt-stack issue page, pipeline table steps 1-3 and the proxy
 * gate of its "Risks" paragraph; readings in oracle.c).  H f64 [I x I]. */
void qto_hessian_full(const float* X, int64_t T, int64_t I, double* H);
/* U [n x n] f64: the upper Cholesky factor of (H + damp mean(diag H) I)^-1,
 * zeros below the diagonal; 0 or -1 (not positive definite). */
int qto_gptq_factor(const double* H, int64_t n, double damp, double* U);
/* The GPTQ sweep with the int3-g64 rounder; U f32 [I x I]; block a multiple
 * of 64. */
void qto_gptq_i3(const float* W, int64_t O, int64_t I, const float* U, int block,
                 float* scales, int8_t* codes);
/* f64 replay along given codes/scales: column values at decision time and
 * the group bases the algorithm would take. */
void qto_gptq_replay(const float* W, int64_t O, int64_t I, const float* U,
                     const float* scales, const int8_t* codes, double* wt_out,
                     double* base_out);
/* tr(E H E^T) and tr(W H W^T), E = W - s*v. */
void qto_proxy_terms(const float* W, int64_t O, int64_t I, const int8_t* codes,
                     const float* scales, const float* H, double* num, double* den);

#ifdef __cplusplus
}
#endif
#endif
