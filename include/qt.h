/*
 * qt.h -- int3-g64 quantize / pack / dequantize-multiply on MI355X (gfx950).
 *
 * C ABI of libqt.so.  Plain pointers and sizes only; no framework types.
 *
 * Format (the "int3-g64 (fmt=5)" pull request page, section "Design", Layout
 * bullet): a weight matrix W[O x I] (O output rows, I inputs, y = W x) is cut,
 * per row, into G = ceil(I/64) groups of 64 inputs; group g covers columns
 * [64g, min(64g+64, I)) and the last one may be short.  Every group packs to
 * 24 bytes: a 16-byte low plane holding u & 3 and an 8-byte high plane holding
 * u >> 2, where u = v + 4 and the code v lies in [-4, 3].  Inside the planes,
 * value 4b+i of the group sits in bits 2i..2i+1 of low byte b and value 8c+i in
 * bit i of high byte c; the padding slots of a short group hold v = 0.  Groups
 * are stored row-major: group (o, g) starts at byte (o*G + g)*24.  One f32
 * scale per group lives in a separate row-major tensor scales[O x G]; the
 * weight the pair denotes is scales[o,g] * v.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; all tensors are
 *     contiguous and row-major; the caller owns every buffer.  The library
 *     never allocates or frees device memory.  It keeps no mutable global
 *     state, so calls are reentrant, with one exception stated at its
 *     declaration: qt_hessian_diag_noalloc, whose scratch is a device array
 *     shared by its calls on a device.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns before the work completes; results are
 *     valid once the caller has synchronised that stream.
 *   - Arguments are validated on the host first.  On any error nothing is
 *     enqueued and a nonzero qt_status is returned.  A failed launch returns
 *     QT_ERR_LAUNCH.  Faults inside a kernel surface at the caller's next
 *     synchronisation.  No exception crosses this interface.
 *   - Alignment: f32 and int32 buffers 4 bytes, bf16 buffers 2 bytes, int3
 *     `packed` buffers 4 bytes (qt_pack_i3, qt_matvec_i3, qt_matmul_i3,
 *     qt_matvec_i3_grouped).  The int4 calls, qt_gptq_proxy and qt_moe_layer
 *     take `packed` at 16 bytes.
 *     Narrower alignment than the kernels' natural one costs speed, not
 *     correctness: the multiply kernels switch to element loads for inputs
 *     that are not 16-byte aligned, and read 4-byte-aligned packed groups
 *     with multi-dword loads at 4-byte alignment (the unaligned access mode
 *     that the ROCm runtime sets on gfx9 and later).  Outputs must not
 *     overlap inputs (QT_ERR_ALIAS).
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 *   - Results are deterministic: no kernel uses floating-point atomics, and
 *     repeated calls on the same inputs give bit-identical outputs.
 */
#ifndef QT_H
#define QT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QT_OK = 0,
    QT_ERR_NULL = 1,      /* a required pointer is NULL                      */
    QT_ERR_SHAPE = 2,     /* a size is out of range or overflows             */
    QT_ERR_ALIGN = 3,     /* a pointer is not aligned as required            */
    QT_ERR_DTYPE = 4,     /* unsupported element type                        */
    QT_ERR_ARG = 5,       /* another argument is out of range                */
    QT_ERR_ALIAS = 6,     /* an output overlaps an input                     */
    QT_ERR_LAUNCH = 7,    /* the kernel launch failed                        */
    QT_ERR_WORKSPACE = 8, /* workspace missing or too small                  */
    QT_ERR_SCRATCH = 9    /* larger than the built-in scratch (_noalloc)     */
} qt_status;

typedef enum { QT_F32 = 0, QT_BF16 = 1 } qt_dtype;

/* Largest I accepted by every entry point (columns are indexed in 32 bits). */
#define QT_MAX_I 2147483647LL

/* Host: number of groups per row, ceil(I/64) (0 for I < 1). */
int64_t qt_groups(int64_t I);

/* Host: bytes of the packed weights of an O x I matrix, O*ceil(I/64)*24
 * (the byte count stated on the pull request page's format-detection
 * comment).  0 for a non-positive size. */
int64_t qt_packed_bytes(int64_t O, int64_t I);

/* Host: human-readable name of a status code (static storage). */
const char* qt_status_str(qt_status s);

/*
 * Importance weights: d[j] = sum_t X[t,j]^2, the diagonal of H = sum X^T X
 * (the tt-stack issue page, pipeline table step 1: H accumulated per linear
 * input over the calibration tokens, fp32 accumulation on the device).
 *   X          [T x I], element type xt (QT_F32 or QT_BF16)
 *   d          [I] f32 output; accumulate = 0: d = sum, 1: d += sum
 *   workspace  device scratch of at least qt_hessian_workspace_bytes(T, I)
 *              bytes (4-byte aligned); may be NULL when that size is 0
 * Partial sums over token slabs go to the workspace and are added in a fixed
 * order, so the result does not depend on scheduling.
 */
size_t qt_hessian_workspace_bytes(int64_t T, int64_t I);
qt_status qt_hessian_diag(const void* X, qt_dtype xt, int64_t T, int64_t I,
                          float* d, int accumulate, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * qt_hessian_diag for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments minus the workspace, same kernels and summation order, so
 * the result is bit-identical to qt_hessian_diag's.  The slab partials live
 * in a file-scope device array of qt_hessian_scratch_bytes() bytes (16 MiB)
 * that each device holds until the process ends; its device address is
 * taken once per device, with that device current, on the first call there
 * (`stream` must belong to the current device).  Nothing is allocated or
 * freed by any call.  Problems whose qt_hessian_workspace_bytes(T, I)
 * exceeds that size return QT_ERR_SCRATCH with nothing enqueued (at the
 * largest slab count, 128, that is I > 32768).  Every call on a device uses
 * the same array: calls that overlap in time on one device (other streams,
 * other threads) race on it and must be ordered by the caller.  The array
 * needs no clearing: every partial is written before it is read.
 */
size_t qt_hessian_scratch_bytes(void);
qt_status qt_hessian_diag_noalloc(const void* X, qt_dtype xt, int64_t T, int64_t I,
                                  float* d, int accumulate, void* stream);

/*
 * Per-group scale choice and code emission (pull request page, "Why this
 * format" item 1: a 3-bit group-64 absmax quantizer; NeUQI accuracy page,
 * first paragraph: a grid search over scales weighted by activation
 * importance).  For every group with real values w_j (j < n):
 *   base = max_j |w_j| * 0.25                              (f32)
 *   candidate k: s_k = base * f_k, f_k = f32(lo + k*(hi-lo)/(n_grid-1)),
 *                f_{n_grid-1} = hi; with n_grid = 0 the single candidate
 *                is s = base
 *   q_j(s) = 0 if s == 0, else clamp(rne(w_j / s), -4, 3)  (IEEE division)
 *   E_k = sum_j d_j * (w_j - s_k*q_j)^2, every operation a rounded f32
 *         operation without fused multiply-add, summed by halving
 *         (a[j] += a[j+m] for m = 32, 16, ..., 1 over the 64 slots, padding
 *         slots contributing 0)
 *   k* = the smallest k with the least E_k
 * Outputs scales[o,g] = s_{k*}, codes[o, 64g+j] = q_j(s_{k*}),
 * grid_idx[o,g] = k*.  Codes, scales and k* are bit-exact functions of the
 * inputs.
 *   W        [O x I] f32
 *   d        [I] f32 importance (>= 0), or NULL for all ones
 *   n_grid   0, or 2..256 candidates; lo, hi with 0 < lo <= hi (ignored for 0)
 *   scales   [O x G] f32 out; codes [O x I] int8 out;
 *   grid_idx [O x G] uint8 out, or NULL
 */
qt_status qt_quantize_g64(const float* W, int64_t O, int64_t I, const float* d,
                          int32_t n_grid, float lo, float hi, float* scales,
                          int8_t* codes, uint8_t* grid_idx, void* stream);

/*
 * Two-stage signed scale search (NeUQI accuracy page, first paragraph:
 * symmetric layers use a two-stage signed scale search; results notes: 64/32
 * points by default).  Objective, rounding, codes and tie rule as
 * qt_quantize_g64; the candidates are
 *   stage 1: s = +base*f_k and -base*f_k for k = 0..n1-1 (order: k
 *            ascending, + before -), f_k the n1-point grid of [lo, hi];
 *   stage 2: n2 points t_j of [f_{k1-1}, f_{k1+1}] around the stage-1
 *            winner k1 (clipped to the grid ends), t_j formed like the grid,
 *            with the winner's sign;
 * and the result is the strict minimum over [stage-1 winner, t_0 .. t_{n2-1}]
 * (ties keep the earlier candidate).  A negative scale lets the largest |w|
 * take the -4 level.  Scales may be negative; codes and scales are bit-exact
 * functions of the inputs.
 *   n1  2..256; n2 0 (stage 1 only) or 2..256; lo, hi with 0 < lo <= hi
 *   other arguments as qt_quantize_g64 (no grid index output)
 */
qt_status qt_quantize_g64_signed(const float* W, int64_t O, int64_t I, const float* d,
                                 int32_t n1, int32_t n2, float lo, float hi, float* scales,
                                 int8_t* codes, void* stream);

/*
 * Bit-plane packer (pull request page, "Design", Layout bullet): codes
 * [O x I] int8 in [-4, 3] -> packed [O*G*24] bytes in the layout described at
 * the top of this header, short groups padded with v = 0.  Codes outside
 * [-4, 3] are masked to their low 3 bits of v + 4.
 */
qt_status qt_pack_i3(const int8_t* codes, int64_t O, int64_t I,
                     uint8_t* packed, void* stream);

/*
 * Dequantize-and-multiply, one vector (pull request page, "Design", Kernel
 * bullet: an exact-f32 path with per-group scale accumulation):
 *   y[o] = sum_g scales[o,g] * sum_{j<n_g} v[o,64g+j] * x[64g+j]
 * computed in f32 (products and sums rounded in f32; agreement with the fp64
 * dequantize-then-multiply value is within 1e-5 of sum_i |w_oi * x_i|).
 *   packed [O*G*24], scales [O x G] f32, x [I] f32, y [O] f32 out.
 */
qt_status qt_matvec_i3(const uint8_t* packed, const float* scales, int64_t O,
                       int64_t I, const float* x, float* y, void* stream);

/*
 * Dequantize-and-multiply, a batch: Y[t,o] = sum_i X[t,i] * w[o,i], t < B.
 *   X [B x I] of type xt, Y [B x O] f32 out.
 *   xt == QT_F32, or B < 16: the exact-f32 path of qt_matvec_i3 (bf16 inputs
 *     are widened exactly to f32); tolerance 1e-5 as above.
 *   xt == QT_BF16 and B >= 16: MFMA path.  The codes enter the matrix cores
 *     as exact bf16 values, each 64-input group is reduced in f32 and then
 *     scaled by its f32 scale; tolerance 2e-3 of sum_i |w_oi * X_ti|.
 */
qt_status qt_matmul_i3(const uint8_t* packed, const float* scales, int64_t O,
                       int64_t I, const void* X, qt_dtype xt, int64_t B,
                       float* Y, void* stream);

/*
 * Grouped dequantize-and-multiply for mixture-of-experts decode (the pull
 * request page's setting: every routed expert's weights are read once per
 * step).  E experts of identical shape O x I, stored back to back:
 *   packed  [E][O*G*24], scales [E][O x G]
 *   pairs p = 0..P-1 are sorted by expert; the pairs of expert e are
 *   p in [expert_offsets[e], expert_offsets[e+1]); expert_offsets [E+1]
 *   int32 on the device with expert_offsets[0] = 0, nondecreasing,
 *   expert_offsets[E] = P.
 *   X       input rows; row of pair p is X[pair_row[p]] when pair_row is
 *           not NULL (int32 [P], values in [0, n_x_rows)), else X[p].
 *   Y       [P x O] f32 out: Y[p] = W_{e(p)} X[row(p)], tolerance 1e-5 as
 *           qt_matvec_i3.  The products are formed on the matrix cores from
 *           the exact codes and an exact split of each f32 input into three
 *           bf16 pieces, and every group is summed in f32 and scaled by its
 *           f32 scale.
 * Everything runs in one launch; experts with no pair cost no weight reads.
 */
qt_status qt_matvec_i3_grouped(const uint8_t* packed, const float* scales,
                               int32_t E, int64_t O, int64_t I,
                               const float* X, int64_t n_x_rows,
                               const int32_t* pair_row,
                               const int32_t* expert_offsets, int32_t P,
                               float* Y, void* stream);

/*
 * Grouped int4 (the pull request page's discussion: group-scaled int4 took
 * its own format number beside int3-g64 and carries the same O*ceil(I/64)
 * scale count; the per-projection ablation table lists int4-g64 and
 * int4-g64-up3, experts at grouped int4 with up_proj at int3-g64).  The page
 * prints no layout; this library reads it as:
 *   the 4-bit symmetric quantizer per 64-input group: base = absmax * 0.125,
 *   codes v in [-8, 7]; every group packs to 32 bytes of u = v + 8, value j
 *   of the group in the low nibble of byte j/2 for even j and in the high
 *   nibble for odd j; short groups padded with v = 0 (u = 8); group (o, g)
 *   starts at byte (o*G + g)*32; scales[O x G] f32 as for int3-g64.
 */

/* Host: bytes of the packed int4 weights, O*ceil(I/64)*32 (0 for a
 * non-positive size). */
int64_t qt_packed_bytes_i4(int64_t O, int64_t I);

/*
 * qt_quantize_g64 for int4 codes: base = max_j |w_j| * 0.125 and
 * q_j(s) = 0 if s == 0, else clamp(rne(w_j / s), -8, 7); candidates,
 * objective, halving sum and tie rule exactly as qt_quantize_g64, and the
 * outputs are bit-exact functions of the inputs.  Arguments as
 * qt_quantize_g64.
 */
qt_status qt_quantize_g64_i4(const float* W, int64_t O, int64_t I, const float* d,
                             int32_t n_grid, float lo, float hi, float* scales,
                             int8_t* codes, uint8_t* grid_idx, void* stream);

/*
 * Nibble packer: codes [O x I] int8 in [-8, 7] -> packed [O*G*32] bytes in
 * the layout above.  Codes outside [-8, 7] are masked to the low 4 bits of
 * v + 8.
 */
qt_status qt_pack_i4(const int8_t* codes, int64_t O, int64_t I,
                     uint8_t* packed, void* stream);

/*
 * qt_matvec_i3 on int4 weights: y[o] = sum_g scales[o,g] * sum_j v * x in
 * f32 with per-group scale accumulation; tolerance 1e-5 of sum_i |w_oi x_i|.
 *   packed [O*G*32], scales [O x G] f32, x [I] f32, y [O] f32 out.
 */
qt_status qt_matvec_i4(const uint8_t* packed, const float* scales, int64_t O,
                       int64_t I, const float* x, float* y, void* stream);

/*
 * qt_matmul_i3 on int4 weights, every batch size on the exact-f32 path (bf16
 * inputs widened exactly); tolerance 1e-5 of sum_i |w_oi X_ti|.
 *   X [B x I] of type xt (B >= 1), Y [B x O] f32 out.
 */
qt_status qt_matmul_i4(const uint8_t* packed, const float* scales, int64_t O,
                       int64_t I, const void* X, qt_dtype xt, int64_t B,
                       float* Y, void* stream);

/*
 * qt_matvec_i3_grouped on grouped int4 experts (packed [E][O*G*32]); the
 * per-projection mix of the ablation table (experts at int4 with up_proj at
 * int3-g64) calls qt_matvec_i3_grouped for the int3 projection and this for
 * the others.  Arguments, routing layout and tolerance as
 * qt_matvec_i3_grouped; the int4 codes enter the matrix cores as exact bf16
 * values of v/16 and the result is scaled back by 16 (exact).
 */
qt_status qt_matvec_i4_grouped(const uint8_t* packed, const float* scales,
                               int32_t E, int64_t O, int64_t I,
                               const float* X, int64_t n_x_rows,
                               const int32_t* pair_row,
                               const int32_t* expert_offsets, int32_t P,
                               float* Y, void* stream);

/*
 * GPTQ with the int3-g64 rounder (the tt-stack issue page, pipeline table:
 * step 1 the full H = sum_t X^T X per linear input, fp32 accumulation on the
 * device; step 2 a Cholesky / inverse of H; step 3 the GPTQ/LDLQ column
 * sweep, serial rounding inside 128-column blocks and then the matmul
 * W[:, rest] -= E Hinv[blk, rest]; the "Risks" paragraph's proxy error
 * tr(E H E^T) / tr(W H W^T)).  The page prints no formulas; this library
 * reads them as:
 *   A = H + damp * mean(diag H) * I;  U = the upper Cholesky factor of A^-1;
 *   per row, column by column: at a group's first column the group scale
 *   s = absmax/4 of the group's current values; q = clamp(rne(w/s), -4, 3)
 *   (IEEE division; 0 when s == 0); err = (w - s q) / U[i][i]; every later
 *   column j takes w_j -= err U[i][j] (inside a 128-column block one fused
 *   multiply-add per update in column order; from one block to the later
 *   columns a matrix product in f32 on the matrix cores).
 */

/*
 * Full Hessian: H [I x I] f32 (both triangles, exactly symmetric) = sum over
 * the T rows of X of x^T x, or H += that (accumulate = 1).  X [T x I] f32 or
 * bf16 (16-byte aligned).  bf16 products are exact (f32 sums); f32 inputs use
 * the f32 matrix cores.  workspace: qt_hessian_full_workspace_bytes(T, I, xt)
 * bytes (16-byte aligned; holds the transposed, padded X).  I <= 8388352.
 */
size_t qt_hessian_full_workspace_bytes(int64_t T, int64_t I, qt_dtype xt);
qt_status qt_hessian_full(const void* X, qt_dtype xt, int64_t T, int64_t I, float* H,
                          int accumulate, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * GPTQ factor: U [I x I] f32 = the upper Cholesky factor of
 * (H + damp * mean(diag H) * I)^-1 (zeros below the diagonal), computed in
 * f64 on the device.  *info (device int32) = 0 on success, else the 1-based
 * index of the first non-positive pivot of the reversed matrix (the result is
 * then not a factor of A).  damp >= 0 (0.01 is the usual choice).
 * workspace: qt_gptq_factor_workspace_bytes(I) bytes (about 8 I^2).
 * I <= 65535.
 */
size_t qt_gptq_factor_workspace_bytes(int64_t I);
qt_status qt_gptq_factor(const float* H, int64_t I, double damp, float* U,
                         int32_t* info, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * GPTQ sweep: W [O x I] f32 (not modified), U from qt_gptq_factor ->
 * scales [O x G] f32 and codes [O x I] int8 in [-4, 3] (pack with
 * qt_pack_i3).  Inside a 128-column block the arithmetic is the exact f32
 * sequence stated above (a sweep with I <= 128 is bit-exact against it); the
 * propagation between blocks sums in f32, so codes near a rounding boundary
 * may differ from another implementation's.  workspace:
 * qt_gptq_workspace_bytes(O, I) bytes (the current weights and the scaled
 * errors of four blocks, about (O*I + 512*O) * 4).
 */
size_t qt_gptq_workspace_bytes(int64_t O, int64_t I);
qt_status qt_gptq_i3(const float* W, int64_t O, int64_t I, const float* U,
                     float* scales, int8_t* codes, void* workspace,
                     size_t ws_bytes, void* stream);

/*
 * Proxy error terms: terms[0] = tr(E H E^T), terms[1] = tr(W H W^T) (device
 * f64 [2]) with E = W - s*v, the packed int3-g64 weights decoded; products on
 * the f32 matrix cores, per-row partials and totals summed in a fixed order.
 * The gate's ratio is terms[0] / terms[1].  workspace:
 * qt_gptq_proxy_workspace_bytes(O, I) bytes; 2*O and I padded to 128 must not
 * exceed 65535.
 */
size_t qt_gptq_proxy_workspace_bytes(int64_t O, int64_t I);
qt_status qt_gptq_proxy(const float* W, const uint8_t* packed, const float* scales,
                        int64_t O, int64_t I, const float* H, double* terms,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * Mixture-of-experts expert layer, as five launches on the stream: a
 * one-block routing, the gate and up projections (one grouped launch), h =
 * SwiGLU(g, u), the down projection (the grouped launch) and the combine of
 * each token's experts (the pull request page's MoE decode setting; its
 * per-projection ablation names gate_proj, up_proj and down_proj, each at
 * int3-g64 or grouped int4).  The pages give no expert formula or combine
 * rule; this library reads them as
 *   experts of token t: the k largest logits[t] (equal logits: lower expert
 *   index first); weights w_tj = softmax over those k logits (f32);
 *   y_e(x) = W_down,e (silu(W_gate,e x) * (W_up,e x)), silu(z) = z/(1+e^-z);
 *   out[t] = sum_j w_tj y_{e_tj}(x_t), j in descending-logit order.
 * Each projection is the grouped multiply (exact codes and exact 3-piece
 * splits of the f32 inputs on the matrix cores, f32 per-group sums).
 *   X [T x D] f32 (16-byte aligned), logits [T x E] f32; experts stored back
 *   to back: gate, up [E][F x D], down [E][D x F], each packed in its format
 *   (bits 3: 24-byte int3-g64 groups, 4: 32-byte grouped int4) with scales
 *   [E][rows x cols/64]; out [T x D] f32 (16-byte aligned).
 *   D and F multiples of 128; 1 <= k <= min(32, E); E <= 512; T <= 2^22.
 *   workspace: qt_moe_layer_workspace_bytes(T, k, E, D, F) bytes (the f32
 *   products g, u, h and the down outputs, (T k)(3F + D) * 4, plus the
 *   routing tables).
 * Every output is written once, in a fixed order: results are deterministic.
 */
size_t qt_moe_layer_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t D, int64_t F);
qt_status qt_moe_layer(const float* X, int64_t T, int64_t D, int64_t F, const float* logits,
                       int32_t E, int32_t k, const uint8_t* gate_packed,
                       const float* gate_scales, int32_t gate_bits,
                       const uint8_t* up_packed, const float* up_scales, int32_t up_bits,
                       const uint8_t* down_packed, const float* down_scales,
                       int32_t down_bits, float* out, void* workspace, size_t ws_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QT_H */
