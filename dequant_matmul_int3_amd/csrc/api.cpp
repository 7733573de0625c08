// C-ABI layer of libqt.so: host-side argument validation, then one launch
// (or a short fixed sequence of launches) on the caller's stream.  See qt.h
// for the contract of every entry point.
#include <cmath>
#include "qt.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qt_internal.h"

namespace {

using qt::kGroup;
using qt::kGroupBytes;
using qt::kGroupBytesI4;

// Overflow-checked product a*b*c of non-negative sizes; -1 on overflow.
int64_t mul3(int64_t a, int64_t b, int64_t c) {
    __int128 p = (__int128)a * b * c;
    if (p > INT64_MAX) return -1;
    return (int64_t)p;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Byte ranges [p, p+n) and [q, q+m) overlap.
bool overlap(const void* p, int64_t n, const void* q, int64_t m) {
    if (!p || !q || n <= 0 || m <= 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

// gbytes: packed bytes per group (24 for int3, 32 for int4)
qt_status shape_ok(int64_t O, int64_t I, int64_t gbytes = kGroupBytes) {
    if (O < 1 || I < 1 || I > QT_MAX_I) return QT_ERR_SHAPE;
    if (mul3(O, (I + kGroup - 1) / kGroup, gbytes) < 0 || mul3(O, I, 4) < 0)
        return QT_ERR_SHAPE;
    return QT_OK;
}

qt_status launched(hipError_t e) { return e == hipSuccess ? QT_OK : QT_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int64_t qt_groups(int64_t I) { return I < 1 ? 0 : (I - 1) / kGroup + 1; }  // no overflow at INT64_MAX

int64_t qt_packed_bytes(int64_t O, int64_t I) {
    if (O < 1 || I < 1) return 0;
    const int64_t b = mul3(O, qt_groups(I), kGroupBytes);
    return b < 0 ? 0 : b;
}

int64_t qt_packed_bytes_i4(int64_t O, int64_t I) {
    if (O < 1 || I < 1) return 0;
    const int64_t b = mul3(O, qt_groups(I), kGroupBytesI4);
    return b < 0 ? 0 : b;
}

const char* qt_status_str(qt_status s) {
    switch (s) {
        case QT_OK: return "ok";
        case QT_ERR_NULL: return "a required pointer is NULL";
        case QT_ERR_SHAPE: return "a size is out of range";
        case QT_ERR_ALIGN: return "a pointer is misaligned";
        case QT_ERR_DTYPE: return "unsupported element type";
        case QT_ERR_ARG: return "an argument is out of range";
        case QT_ERR_ALIAS: return "an output overlaps an input";
        case QT_ERR_LAUNCH: return "kernel launch failed";
        case QT_ERR_WORKSPACE: return "workspace missing or too small";
        case QT_ERR_SCRATCH: return "problem larger than the built-in scratch";
    }
    return "unknown status";
}

size_t qt_hessian_workspace_bytes(int64_t T, int64_t I) {
    if (T < 1 || I < 1 || I > QT_MAX_I) return 0;
    const int slabs = qt::hessian_slabs(T, I);
    if (slabs <= 1) return 0;
    const int64_t b = mul3(slabs, I, 4);
    return b < 0 ? 0 : (size_t)b;
}

qt_status qt_hessian_diag(const void* X, qt_dtype xt, int64_t T, int64_t I, float* d,
                          int accumulate, void* workspace, size_t ws_bytes, void* stream) {
    if (!X || !d) return QT_ERR_NULL;
    if (xt != QT_F32 && xt != QT_BF16) return QT_ERR_DTYPE;
    if (T < 1 || I < 1 || I > QT_MAX_I) return QT_ERR_SHAPE;
    const int64_t esz = xt == QT_F32 ? 4 : 2;
    const int64_t xbytes = mul3(T, I, esz);
    if (xbytes < 0) return QT_ERR_SHAPE;
    if (accumulate != 0 && accumulate != 1) return QT_ERR_ARG;
    if (!aligned(X, (uintptr_t)esz) || !aligned(d, 4)) return QT_ERR_ALIGN;
    const size_t need = qt_hessian_workspace_bytes(T, I);
    if (need > 0) {
        if (!workspace || ws_bytes < need) return QT_ERR_WORKSPACE;
        if (!aligned(workspace, 4)) return QT_ERR_ALIGN;
    }
    if (overlap(d, I * 4, X, xbytes)) return QT_ERR_ALIAS;
    if (need > 0 && (overlap(workspace, (int64_t)need, X, xbytes) ||
                     overlap(workspace, (int64_t)need, d, I * 4)))
        return QT_ERR_ALIAS;
    return launched(qt::launch_hessian_diag(X, xt == QT_BF16, T, I, d, accumulate,
                                            static_cast<float*>(workspace), as_stream(stream)));
}

qt_status qt_hessian_diag_noalloc(const void* X, qt_dtype xt, int64_t T, int64_t I, float* d,
                                  int accumulate, void* stream) {
    if (!X || !d) return QT_ERR_NULL;
    if (xt != QT_F32 && xt != QT_BF16) return QT_ERR_DTYPE;
    if (T < 1 || I < 1 || I > QT_MAX_I) return QT_ERR_SHAPE;
    const int64_t esz = xt == QT_F32 ? 4 : 2;
    const int64_t xbytes = mul3(T, I, esz);
    if (xbytes < 0) return QT_ERR_SHAPE;
    if (accumulate != 0 && accumulate != 1) return QT_ERR_ARG;
    if (!aligned(X, (uintptr_t)esz) || !aligned(d, 4)) return QT_ERR_ALIGN;
    const size_t need = qt_hessian_workspace_bytes(T, I);
    if (need > qt::kHessianScratchBytes) return QT_ERR_SCRATCH;
    if (overlap(d, I * 4, X, xbytes)) return QT_ERR_ALIAS;
    float* ws = nullptr;
    if (need > 0) {
        ws = static_cast<float*>(qt::hessian_scratch_ptr());
        if (!ws) return QT_ERR_LAUNCH;
    }
    return launched(qt::launch_hessian_diag(X, xt == QT_BF16, T, I, d, accumulate, ws,
                                            as_stream(stream)));
}

size_t qt_hessian_scratch_bytes(void) { return qt::kHessianScratchBytes; }

namespace {

// Candidate factors: n_grid equally spaced points of [lo, hi], formed in
// double and rounded once; the last one is hi itself.  n_grid == 0 is the
// single plain absmax/2^(b-1) scale (factor 1).  half = 2^(b-1): 4 for int3,
// 8 for int4.
int make_grid(int32_t n_grid, float lo, float hi, qt::GridTable& tab, double half = 4.0) {
    int ncand = 1;
    if (n_grid == 0) {
        tab.f[0] = 1.0f;
    } else {
        ncand = n_grid;
        const double step = ((double)hi - (double)lo) / (double)(n_grid - 1);
        for (int k = 0; k < n_grid; ++k) tab.f[k] = (float)((double)lo + (double)k * step);
        tab.f[n_grid - 1] = hi;
    }
    // In a group with a normal base = absmax/half and s = fl(base * f), every
    // |w/s| stays below bound = half/f * (1 + 2^-20).  The kernel accepts
    // rint(w * rcp(s)) when that quotient lies closer than margin to its
    // nearest integer, margin = 0.5 - 2^-21 * bound rounded toward zero: twice
    // the combined error of the reciprocal quotient and of fl(w/s).  Huge
    // quotient ranges get margin 0, which sends every lane to the division.
    for (int k = 0; k < ncand; ++k) {
        const double bound = half / (double)tab.f[k] * (1.0 + 0x1p-20);
        if (!(bound < 0x1p20)) {
            tab.margin[k] = 0.0f;
            continue;
        }
        const double m = 0.5 - bound * 0x1p-21;
        float mf = (float)m;
        if ((double)mf > m) mf = std::nextafter(mf, 0.0f);
        tab.margin[k] = mf;
    }
    tab.fmin = tab.f[0];
    tab.fmax = tab.f[ncand - 1];
    return ncand;
}

qt_status quantize_args_ok(const float* W, int64_t O, int64_t I, const float* d,
                           const float* scales, const int8_t* codes, const uint8_t* grid_idx) {
    if (!W || !scales || !codes) return QT_ERR_NULL;
    qt_status st = shape_ok(O, I, kGroupBytesI4);
    if (st != QT_OK) return st;
    if (!aligned(W, 4) || !aligned(scales, 4) || (d && !aligned(d, 4))) return QT_ERR_ALIGN;
    const int64_t G = qt_groups(I);
    const int64_t wb = O * I * 4, sb = O * G * 4, cb = O * I, gb = O * G;
    if (overlap(scales, sb, W, wb) || overlap(codes, cb, W, wb) ||
        overlap(scales, sb, codes, cb) || (d && (overlap(scales, sb, d, I * 4) ||
                                                 overlap(codes, cb, d, I * 4))) ||
        (grid_idx && (overlap(grid_idx, gb, W, wb) || overlap(grid_idx, gb, scales, sb) ||
                      overlap(grid_idx, gb, codes, cb) || (d && overlap(grid_idx, gb, d, I * 4)))))
        return QT_ERR_ALIAS;
    return QT_OK;
}

bool grid_ok(float lo, float hi) { return lo > 0.0f && lo <= hi && hi < __builtin_inff(); }

}  // namespace

qt_status qt_quantize_g64(const float* W, int64_t O, int64_t I, const float* d, int32_t n_grid,
                          float lo, float hi, float* scales, int8_t* codes, uint8_t* grid_idx,
                          void* stream) {
    qt_status st = quantize_args_ok(W, O, I, d, scales, codes, grid_idx);
    if (st != QT_OK) return st;
    if (n_grid != 0 && (n_grid < 2 || n_grid > qt::kMaxGrid)) return QT_ERR_ARG;
    if (n_grid != 0 && !grid_ok(lo, hi)) return QT_ERR_ARG;
    qt::GridTable tab{};
    const int ncand = make_grid(n_grid, lo, hi, tab);
    return launched(qt::launch_quantize_g64(W, O, I, d, ncand, 0, false, 3, tab, scales, codes,
                                            grid_idx, as_stream(stream)));
}

qt_status qt_quantize_g64_i4(const float* W, int64_t O, int64_t I, const float* d,
                             int32_t n_grid, float lo, float hi, float* scales, int8_t* codes,
                             uint8_t* grid_idx, void* stream) {
    qt_status st = quantize_args_ok(W, O, I, d, scales, codes, grid_idx);
    if (st != QT_OK) return st;
    if (n_grid != 0 && (n_grid < 2 || n_grid > qt::kMaxGrid)) return QT_ERR_ARG;
    if (n_grid != 0 && !grid_ok(lo, hi)) return QT_ERR_ARG;
    qt::GridTable tab{};
    const int ncand = make_grid(n_grid, lo, hi, tab, 8.0);
    return launched(qt::launch_quantize_g64(W, O, I, d, ncand, 0, false, 4, tab, scales, codes,
                                            grid_idx, as_stream(stream)));
}

qt_status qt_quantize_g64_signed(const float* W, int64_t O, int64_t I, const float* d,
                                 int32_t n1, int32_t n2, float lo, float hi, float* scales,
                                 int8_t* codes, void* stream) {
    qt_status st = quantize_args_ok(W, O, I, d, scales, codes, nullptr);
    if (st != QT_OK) return st;
    if (n1 < 2 || n1 > qt::kMaxGrid) return QT_ERR_ARG;
    if (n2 != 0 && (n2 < 2 || n2 > qt::kMaxGrid)) return QT_ERR_ARG;
    if (!grid_ok(lo, hi)) return QT_ERR_ARG;
    qt::GridTable tab{};
    const int ncand = make_grid(n1, lo, hi, tab);
    return launched(qt::launch_quantize_g64(W, O, I, d, ncand, n2, true, 3, tab, scales, codes,
                                            nullptr, as_stream(stream)));
}

qt_status qt_pack_i3(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed, void* stream) {
    if (!codes || !packed) return QT_ERR_NULL;
    qt_status st = shape_ok(O, I);
    if (st != QT_OK) return st;
    if (!aligned(packed, 4)) return QT_ERR_ALIGN;
    if (overlap(packed, qt_packed_bytes(O, I), codes, O * I)) return QT_ERR_ALIAS;
    return launched(qt::launch_pack_i3(codes, O, I, packed, as_stream(stream)));
}

qt_status qt_pack_i4(const int8_t* codes, int64_t O, int64_t I, uint8_t* packed, void* stream) {
    if (!codes || !packed) return QT_ERR_NULL;
    qt_status st = shape_ok(O, I, kGroupBytesI4);
    if (st != QT_OK) return st;
    if (!aligned(packed, 16)) return QT_ERR_ALIGN;
    if (overlap(packed, qt_packed_bytes_i4(O, I), codes, O * I)) return QT_ERR_ALIAS;
    return launched(qt::launch_pack_i4(codes, O, I, packed, as_stream(stream)));
}

namespace {

qt_status matvec_bits(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                      const float* x, float* y, void* stream, int bits) {
    if (!packed || !scales || !x || !y) return QT_ERR_NULL;
    const int64_t gbytes = bits == 3 ? kGroupBytes : kGroupBytesI4;
    qt_status st = shape_ok(O, I, gbytes);
    if (st != QT_OK) return st;
    if (!aligned(packed, bits == 3 ? 4 : 16) || !aligned(scales, 4) || !aligned(x, 4) ||
        !aligned(y, 4))
        return QT_ERR_ALIGN;
    const int64_t G = qt_groups(I);
    if (overlap(y, O * 4, packed, O * G * gbytes) || overlap(y, O * 4, scales, O * G * 4) ||
        overlap(y, O * 4, x, I * 4))
        return QT_ERR_ALIAS;
    return launched(qt::launch_gemv_batch(packed, scales, O, I, x, false, 1, y,
                                          as_stream(stream), bits));
}

}  // namespace

qt_status qt_matvec_i3(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                       const float* x, float* y, void* stream) {
    return matvec_bits(packed, scales, O, I, x, y, stream, 3);
}

qt_status qt_matvec_i4(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                       const float* x, float* y, void* stream) {
    return matvec_bits(packed, scales, O, I, x, y, stream, 4);
}

qt_status qt_matmul_i4(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                       const void* X, qt_dtype xt, int64_t B, float* Y, void* stream) {
    if (!packed || !scales || !X || !Y) return QT_ERR_NULL;
    if (xt != QT_F32 && xt != QT_BF16) return QT_ERR_DTYPE;
    qt_status st = shape_ok(O, I, kGroupBytesI4);
    if (st != QT_OK) return st;
    if (B < 1) return QT_ERR_SHAPE;
    const int64_t esz = xt == QT_F32 ? 4 : 2;
    const int64_t xb = mul3(B, I, esz), yb = mul3(B, O, 4);
    if (xb < 0 || yb < 0) return QT_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(Y, 4)) return QT_ERR_ALIGN;
    if (!aligned(X, (uintptr_t)esz)) return QT_ERR_ALIGN;
    const int64_t G = qt_groups(I);
    if (overlap(Y, yb, packed, O * G * kGroupBytesI4) || overlap(Y, yb, scales, O * G * 4) ||
        overlap(Y, yb, X, xb))
        return QT_ERR_ALIAS;
    return launched(qt::launch_gemv_batch(packed, scales, O, I, X, xt == QT_BF16, B, Y,
                                          as_stream(stream), 4));
}

qt_status qt_matmul_i3(const uint8_t* packed, const float* scales, int64_t O, int64_t I,
                       const void* X, qt_dtype xt, int64_t B, float* Y, void* stream) {
    if (!packed || !scales || !X || !Y) return QT_ERR_NULL;
    if (xt != QT_F32 && xt != QT_BF16) return QT_ERR_DTYPE;
    qt_status st = shape_ok(O, I);
    if (st != QT_OK) return st;
    // the MFMA grid has one block row per 128 tokens (65535 rows at most)
    if (B < 1 || B > 65535LL * 128) return QT_ERR_SHAPE;
    const int64_t esz = xt == QT_F32 ? 4 : 2;
    const int64_t xb = mul3(B, I, esz), yb = mul3(B, O, 4);
    if (xb < 0 || yb < 0) return QT_ERR_SHAPE;
    if (!aligned(packed, 4) || !aligned(scales, 4) || !aligned(Y, 4)) return QT_ERR_ALIGN;
    if (!aligned(X, (uintptr_t)esz)) return QT_ERR_ALIGN;
    const int64_t G = qt_groups(I);
    if (overlap(Y, yb, packed, O * G * kGroupBytes) || overlap(Y, yb, scales, O * G * 4) ||
        overlap(Y, yb, X, xb))
        return QT_ERR_ALIAS;
    if (xt == QT_BF16 && B >= 16)
        return launched(qt::launch_gemm_mfma(packed, scales, O, I,
                                             static_cast<const uint16_t*>(X), B, Y,
                                             as_stream(stream)));
    return launched(qt::launch_gemv_batch(packed, scales, O, I, X, xt == QT_BF16, B, Y,
                                          as_stream(stream)));
}

namespace {

qt_status grouped_bits(const uint8_t* packed, const float* scales, int32_t E, int64_t O,
                       int64_t I, const float* X, int64_t n_x_rows, const int32_t* pair_row,
                       const int32_t* expert_offsets, int32_t P, float* Y, void* stream,
                       int bits) {
    if (!packed || !scales || !X || !expert_offsets || !Y) return QT_ERR_NULL;
    const int64_t gbytes = bits == 3 ? kGroupBytes : kGroupBytesI4;
    qt_status st = shape_ok(O, I, gbytes);
    if (st != QT_OK) return st;
    if (E < 1 || E > 65535 || P < 1 || n_x_rows < 1) return QT_ERR_SHAPE;
    if (!pair_row && n_x_rows < P) return QT_ERR_SHAPE;
    const int64_t G = qt_groups(I);
    const int64_t pk = mul3(E, O * G, gbytes), sk = mul3(E, O * G, 4);
    const int64_t xb = mul3(n_x_rows, I, 4), yb = mul3(P, O, 4);
    if (pk < 0 || sk < 0 || xb < 0 || yb < 0) return QT_ERR_SHAPE;
    if (!aligned(packed, bits == 3 ? 4 : 16) || !aligned(scales, 4) || !aligned(X, 4) ||
        !aligned(Y, 4) || !aligned(expert_offsets, 4) || (pair_row && !aligned(pair_row, 4)))
        return QT_ERR_ALIGN;
    if (overlap(Y, yb, packed, pk) || overlap(Y, yb, scales, sk) || overlap(Y, yb, X, xb) ||
        overlap(Y, yb, expert_offsets, (int64_t)(E + 1) * 4) ||
        (pair_row && overlap(Y, yb, pair_row, (int64_t)P * 4)))
        return QT_ERR_ALIAS;
    return launched(qt::launch_gemv_grouped(packed, scales, E, O, I, X, n_x_rows, pair_row,
                                            expert_offsets, P, Y, as_stream(stream), bits));
}

}  // namespace

qt_status qt_matvec_i3_grouped(const uint8_t* packed, const float* scales, int32_t E, int64_t O,
                               int64_t I, const float* X, int64_t n_x_rows,
                               const int32_t* pair_row, const int32_t* expert_offsets, int32_t P,
                               float* Y, void* stream) {
    return grouped_bits(packed, scales, E, O, I, X, n_x_rows, pair_row, expert_offsets, P, Y,
                        stream, 3);
}

qt_status qt_matvec_i4_grouped(const uint8_t* packed, const float* scales, int32_t E, int64_t O,
                               int64_t I, const float* X, int64_t n_x_rows,
                               const int32_t* pair_row, const int32_t* expert_offsets, int32_t P,
                               float* Y, void* stream) {
    return grouped_bits(packed, scales, E, O, I, X, n_x_rows, pair_row, expert_offsets, P, Y,
                        stream, 4);
}

// ---------------------------------------------------------------- MoE layer
size_t qt_moe_layer_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t D, int64_t F) {
    if (T < 1 || k < 1 || E < 1 || D < 1 || F < 1) return 0;
    // the layer's own limits, so that T * k and D + 2 F cannot overflow below
    if (T > (1 << 22) || k > 32 || E > 512 || D > QT_MAX_I || F > QT_MAX_I) return 0;
    if (mul3(T * k, D + 2 * F, 4) < 0) return 0;
    return qt::moe_layer_workspace(T, k, E, D, F);
}

qt_status qt_moe_layer(const float* X, int64_t T, int64_t D, int64_t F, const float* logits,
                       int32_t E, int32_t k, const uint8_t* gate_packed,
                       const float* gate_scales, int32_t gate_bits, const uint8_t* up_packed,
                       const float* up_scales, int32_t up_bits, const uint8_t* down_packed,
                       const float* down_scales, int32_t down_bits, float* out,
                       void* workspace, size_t ws_bytes, void* stream) {
    if (!X || !logits || !gate_packed || !gate_scales || !up_packed || !up_scales ||
        !down_packed || !down_scales || !out || !workspace)
        return QT_ERR_NULL;
    if (T < 1 || D < 128 || F < 128 || D % 128 || F % 128 || D > QT_MAX_I || F > QT_MAX_I)
        return QT_ERR_SHAPE;
    if (E < 1 || E > 512 || k < 1 || k > 32 || k > E || T > (1 << 22)) return QT_ERR_SHAPE;
    const int32_t bits[3] = {gate_bits, up_bits, down_bits};
    for (int b : bits)
        if (b != 3 && b != 4) return QT_ERR_ARG;
    const int64_t gb = gate_bits == 3 ? kGroupBytes : kGroupBytesI4;
    const int64_t ub = up_bits == 3 ? kGroupBytes : kGroupBytesI4;
    const int64_t db = down_bits == 3 ? kGroupBytes : kGroupBytesI4;
    const int64_t gpb = mul3(E, F * (D / 64), gb), upb = mul3(E, F * (D / 64), ub);
    const int64_t dpb = mul3(E, D * (F / 64), db);
    const int64_t gsb = mul3(E, F * (D / 64), 4), dsb = mul3(E, D * (F / 64), 4);
    const int64_t xb = mul3(T, D, 4), lb = mul3(T, E, 4);
    if (gpb < 0 || upb < 0 || dpb < 0 || gsb < 0 || dsb < 0 || xb < 0 || lb < 0)
        return QT_ERR_SHAPE;
    const size_t need = qt_moe_layer_workspace_bytes(T, k, E, D, F);
    if (need == 0) return QT_ERR_SHAPE;
    if (ws_bytes < need) return QT_ERR_WORKSPACE;
    if (!aligned(X, 16) || !aligned(out, 16) || !aligned(logits, 4) || !aligned(gate_packed, 16) ||
        !aligned(up_packed, 16) || !aligned(down_packed, 16) || !aligned(gate_scales, 4) ||
        !aligned(up_scales, 4) || !aligned(down_scales, 4) || !aligned(workspace, 16))
        return QT_ERR_ALIGN;
    const void* ins[8] = {X, logits, gate_packed, gate_scales, up_packed, up_scales, down_packed,
                          down_scales};
    const int64_t inb[8] = {xb, lb, gpb, gsb, upb, gsb, dpb, dsb};
    for (int q = 0; q < 8; ++q)
        if (overlap(out, xb, ins[q], inb[q]) || overlap(workspace, (int64_t)need, ins[q], inb[q]))
            return QT_ERR_ALIAS;
    if (overlap(out, xb, workspace, (int64_t)need)) return QT_ERR_ALIAS;
    return launched(qt::launch_moe_layer(X, T, D, F, logits, E, k, gate_packed, gate_scales,
                                         gate_bits, up_packed, up_scales, up_bits, down_packed,
                                         down_scales, down_bits, out, workspace,
                                         as_stream(stream)));
}

// ---------------------------------------------------------------- GPTQ
size_t qt_hessian_full_workspace_bytes(int64_t T, int64_t I, qt_dtype xt) {
    // rows pad to a multiple of 256 and the f32 kernel takes 128-row tiles on
    // a grid of at most 65535 x 65535
    if (T < 1 || I < 1 || I > 32767 * 256LL || (xt != QT_F32 && xt != QT_BF16)) return 0;
    const int64_t b = mul3(qt::hessian_full_rows(I), qt::hessian_full_tokens(T),
                           xt == QT_F32 ? 4 : 2);
    return b < 0 ? 0 : (size_t)b;
}

qt_status qt_hessian_full(const void* X, qt_dtype xt, int64_t T, int64_t I, float* H,
                          int accumulate, void* workspace, size_t ws_bytes, void* stream) {
    if (!X || !H || !workspace) return QT_ERR_NULL;
    if (xt != QT_F32 && xt != QT_BF16) return QT_ERR_DTYPE;
    if (T < 1 || I < 1 || I > 32767 * 256LL) return QT_ERR_SHAPE;
    const int64_t esz = xt == QT_F32 ? 4 : 2;
    const int64_t xb = mul3(T, I, esz), hb = mul3(I, I, 4);
    if (xb < 0 || hb < 0) return QT_ERR_SHAPE;
    if (accumulate != 0 && accumulate != 1) return QT_ERR_ARG;
    const size_t need = qt_hessian_full_workspace_bytes(T, I, xt);
    if (need == 0) return QT_ERR_SHAPE;
    if (ws_bytes < need) return QT_ERR_WORKSPACE;
    if (!aligned(X, 16) || !aligned(H, 4) || !aligned(workspace, 16)) return QT_ERR_ALIGN;
    if (overlap(H, hb, X, xb) || overlap(workspace, (int64_t)need, X, xb) ||
        overlap(workspace, (int64_t)need, H, hb))
        return QT_ERR_ALIAS;
    return launched(qt::launch_hessian_full(X, xt == QT_BF16, T, I, H, accumulate, workspace,
                                            as_stream(stream)));
}

size_t qt_gptq_factor_workspace_bytes(int64_t I) {
    if (I < 1 || I > 65535) return 0;
    return qt::gptq_factor_workspace(I);
}

qt_status qt_gptq_factor(const float* H, int64_t I, double damp, float* U, int32_t* info,
                         void* workspace, size_t ws_bytes, void* stream) {
    if (!H || !U || !info || !workspace) return QT_ERR_NULL;
    if (I < 1 || I > 65535) return QT_ERR_SHAPE;
    if (!(damp >= 0.0) || !(damp < 1e30)) return QT_ERR_ARG;
    const size_t need = qt_gptq_factor_workspace_bytes(I);
    if (ws_bytes < need) return QT_ERR_WORKSPACE;
    if (!aligned(H, 4) || !aligned(U, 4) || !aligned(info, 4) || !aligned(workspace, 16))
        return QT_ERR_ALIGN;
    const int64_t hb = I * I * 4;
    if (overlap(U, hb, H, hb) || overlap(info, 4, H, hb) || overlap(info, 4, U, hb) ||
        overlap(workspace, (int64_t)need, H, hb) || overlap(workspace, (int64_t)need, U, hb) ||
        overlap(workspace, (int64_t)need, info, 4))
        return QT_ERR_ALIAS;
    return launched(qt::launch_gptq_factor(H, I, damp, U, info, workspace, as_stream(stream)));
}

size_t qt_gptq_workspace_bytes(int64_t O, int64_t I) {
    if (O < 1 || I < 1 || I > QT_MAX_I) return 0;
    if (mul3(O, I + 128, 4) < 0) return 0;
    return qt::gptq_workspace(O, I);
}

qt_status qt_gptq_i3(const float* W, int64_t O, int64_t I, const float* U, float* scales,
                     int8_t* codes, void* workspace, size_t ws_bytes, void* stream) {
    if (!W || !U || !scales || !codes || !workspace) return QT_ERR_NULL;
    qt_status st = shape_ok(O, I);
    if (st != QT_OK) return st;
    if (mul3(I, I, 4) < 0 || (O + 63) / 64 > 0x7fffffffLL) return QT_ERR_SHAPE;
    const size_t need = qt_gptq_workspace_bytes(O, I);
    if (need == 0) return QT_ERR_SHAPE;
    if (ws_bytes < need) return QT_ERR_WORKSPACE;
    if (!aligned(W, 4) || !aligned(U, 4) || !aligned(scales, 4) || !aligned(workspace, 16))
        return QT_ERR_ALIGN;
    const int64_t G = qt_groups(I);
    const int64_t wb = O * I * 4, ub = I * I * 4, sb = O * G * 4, cb = O * I;
    const void* outs[3] = {scales, codes, workspace};
    const int64_t ob[3] = {sb, cb, (int64_t)need};
    for (int k = 0; k < 3; ++k)
        if (overlap(outs[k], ob[k], W, wb) || overlap(outs[k], ob[k], U, ub)) return QT_ERR_ALIAS;
    if (overlap(scales, sb, codes, cb) || overlap(scales, sb, workspace, (int64_t)need) ||
        overlap(codes, cb, workspace, (int64_t)need))
        return QT_ERR_ALIAS;
    return launched(qt::launch_gptq_i3(W, O, I, U, scales, codes, workspace, as_stream(stream)));
}

size_t qt_gptq_proxy_workspace_bytes(int64_t O, int64_t I) {
    if (O < 1 || I < 1) return 0;
    const int64_t Mp = qt::proxy_pad(2 * O), Kp = qt::proxy_pad(I);
    if (Mp > 65535 || Kp > 65535) return 0;
    return qt::gptq_proxy_workspace(O, I);
}

qt_status qt_gptq_proxy(const float* W, const uint8_t* packed, const float* scales, int64_t O,
                        int64_t I, const float* H, double* terms, void* workspace,
                        size_t ws_bytes, void* stream) {
    if (!W || !packed || !scales || !H || !terms || !workspace) return QT_ERR_NULL;
    qt_status st = shape_ok(O, I);
    if (st != QT_OK) return st;
    const size_t need = qt_gptq_proxy_workspace_bytes(O, I);
    if (need == 0) return QT_ERR_SHAPE;
    if (ws_bytes < need) return QT_ERR_WORKSPACE;
    if (!aligned(W, 4) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(H, 4) ||
        !aligned(terms, 8) || !aligned(workspace, 16))
        return QT_ERR_ALIGN;
    const int64_t G = qt_groups(I);
    const int64_t ins[4] = {O * I * 4, O * G * kGroupBytes, O * G * 4, I * I * 4};
    const void* inp[4] = {W, packed, scales, H};
    for (int k = 0; k < 4; ++k)
        if (overlap(terms, 16, inp[k], ins[k]) || overlap(workspace, (int64_t)need, inp[k], ins[k]))
            return QT_ERR_ALIAS;
    if (overlap(terms, 16, workspace, (int64_t)need)) return QT_ERR_ALIAS;
    return launched(qt::launch_gptq_proxy(W, packed, scales, O, I, H, terms, workspace,
                                          as_stream(stream)));
}

}  // extern "C"
