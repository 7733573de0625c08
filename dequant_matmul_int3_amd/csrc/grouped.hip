// Grouped (mixture-of-experts) int3-g64 and grouped-int4 dequantize-and-
// multiply on the gfx950 matrix cores, exact-f32 semantics.
//
// Y[p, o] = sum_g s_e[o,g] * sum_{j<64} v_e[o,64g+j] * x_p[64g+j] for every
// routed pair p of expert e: the per-group scale accumulation of the matmul_i3
// kernel ("int3-g64 (fmt=5)" pull request page, "Design", Kernel bullet) with
// f32 inputs.  Mixed per-projection bits (the same page's per-projection
// ablation: experts at grouped int4 with up_proj at int3-g64) run each
// projection through the instantiation of its own format.
//
// Why the matrix cores.  A vector-ALU GEMV spends one FMA per code per token
// on top of the unpacking; with a few tokens per expert that, not the weight
// stream, bounds it.  Here the codes go to the MFMA as exact bf16 values and
// each f32 input is split into three bf16 pieces whose sum is the input:
//   h = x with the low 16 bits cleared,  m = (x - h) likewise,  l = x - h - m
// (x - h has at most 16 significant bits and the last rest at most 8, so all
// three are bf16 numbers and both subtractions are exact; only a third piece
// below the smallest normal number can lose bits, at most 2^-133 absolute).
// Code times piece products are exact in the matrix core's f32 accumulation,
// so every group's dot product is an f32 sum of exact products, as on the
// vector path; the pieces of a token are summed after the groups.
//
// int4 codes enter as v/16: v_cvt_off_f32_i4 turns a two's-complement nibble
// into that f32 value exactly, whose high half is its bf16 encoding; the
// results are multiplied by 16 at the end (exact: a power of two).
//
// Tiling.  A block of 4 waves owns 64 consecutive output rows of one expert;
// wave w multiplies rows [16w, 16w+16) as the A operand (16 rows x 32 inputs
// per MFMA, lane l: row l%16, eight codes of quarter l/16 of the group; for
// int3 in the order 0 4 1 5 2 6 3 7 within each eight, which the table
// unpacking produces without regrouping, and the inputs are staged in the same
// order).  The B operand columns are (token t, piece p) = 3t+p for up to 5
// tokens per pass over the weights.  Weights, scales and inputs advance in
// chunks of groups (8 here, 16 in the expert layer): the next chunk is loaded
// into registers (16-byte loads of each row's contiguous bytes) while the
// current one is multiplied out of LDS.
#include "grouped_tile.h"

namespace qt {
namespace {

// Eight groups per chunk: half the LDS and staging registers of sixteen, so
// four blocks share a CU (at most 128 VGPRs: four waves per SIMD) and hide
// each other's load latency; 4 against 3 blocks measured 0.483 -> 0.475 ms
// for the int3 MoE step and 0.450 -> 0.424 ms at int4.  The int4 kernel for
// unaligned inputs would spill at that limit and keeps three.
constexpr int kGroupedCG = 8;

template <int BITS, bool W16, bool XV>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(BITS == 3 || XV ? 4 : 3))) void gemv_grouped_mfma_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int32_t I,
    int32_t G, const float* __restrict__ X, int64_t n_x_rows,
    const int32_t* __restrict__ pair_row, const int32_t* __restrict__ off, int32_t P,
    float* __restrict__ Y) {
    __shared__ TileLds<Geo<BITS, kGroupedCG>::kWRow, kGroupedCG> lds;
    grouped_tile<BITS, W16, XV>(lds, blockIdx.y, blockIdx.x, packed, scales, O, I, G, X, n_x_rows,
                                pair_row, off, P, Y);
}

}  // namespace

hipError_t launch_gemv_grouped(const uint8_t* packed, const float* scales, int32_t E,
                               int64_t O, int64_t I, const float* X, int64_t n_x_rows,
                               const int32_t* pair_row, const int32_t* expert_offsets,
                               int32_t P, float* Y, hipStream_t s, int bits) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    const dim3 grid((unsigned)((O + kRows - 1) / kRows), (unsigned)E);
    const bool a16 = (reinterpret_cast<uintptr_t>(packed) & 15) == 0;
    const bool xv = (I % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
#define QT_GROUPED(B, W, V)                                                                   \
    hipLaunchKernelGGL((gemv_grouped_mfma_kernel<B, W, V>), grid, dim3(kThreads), 0, s,     \
                       packed, scales, O, (int32_t)I, (int32_t)G, X, n_x_rows, pair_row,  \
                       expert_offsets, P, Y)
    if (bits == 4) {
        if (!a16) return hipErrorInvalidValue;
        if (xv)
            QT_GROUPED(4, true, true);
        else
            QT_GROUPED(4, true, false);
        return hipGetLastError();
    }
    if (bits != 3) return hipErrorInvalidValue;
    const bool w16 = (G % 2 == 0) && a16;
    if (w16 && xv)
        QT_GROUPED(3, true, true);
    else if (w16)
        QT_GROUPED(3, true, false);
    else if (xv)
        QT_GROUPED(3, false, true);
    else
        QT_GROUPED(3, false, false);
#undef QT_GROUPED
    return hipGetLastError();
}

}  // namespace qt
