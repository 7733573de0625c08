// int3-g64 dequantize-and-multiply for batches of bf16 activations on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Y[t,o] = sum_g s[o,g] * sum_{j<64} v[o,64g+j] * X[t,64g+j]
//
// The int3 codes v in [-4,3] are exact in bf16, so each group's 64-term dot
// product is formed by the matrix cores with exact products and f32
// accumulation, then multiplied by the f32 group scale on the vector ALUs and
// added into an f32 accumulator: the per-group scale accumulation of the
// matmul_i3 kernel ("int3-g64 (fmt=5)" pull request page, "Design", Kernel
// bullet), with bf16 inputs.
//
// Tiling.  A block of 8 waves (two per SIMD) computes a BM = 256 (tokens) x
// BN = 144 (output rows) tile and walks the input dimension one 64-wide group
// at a time; wave w owns tokens [32w, 32w+32) against all 144 rows (2 x 9 MFMA
// tiles of 16x16, two 32-deep MFMAs per tile and group).
//   * Weights: the group's 144 x 64 codes are dequantized once per block into
//     LDS as bf16 (one 16-code quarter per task: byte-parallel unpack, then
//     v_perm_b32 table lookups), with the 144 scales; every wave reads its B
//     operands from there.  The tile is laid out in operand order: the 16 B
//     that lane l takes for row tile nt and 32-deep step ks sit at slot
//     (2 nt + ks) * 64 + l, so each operand read is one contiguous 1 KB, and
//     wave w dequantizes row tile w, 16 lanes per contiguous 256 B.
//   * Activations never touch LDS: each lane loads its A-operand slices
//     (8 consecutive bf16 of one token) straight from global memory into
//     registers with buffer loads, two groups ahead (one on the element-load
//     path for unaligned rows).  Tokens past the batch and
//     inputs past the row use an offset outside the buffer, for which the
//     hardware returns zeros.
// Double-buffered LDS, one barrier per group; packed weights are fetched two
// groups ahead.
//
// For B x O shapes that are not multiples of the tile, out-of-range rows read
// a valid row (their results are discarded) and are never stored.
#include "lds_barrier.h"
#include "qt_internal.h"

namespace qt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int BM = 256;                 // tokens per block tile
constexpr int BN = 144;                 // output rows per block tile (9 x 16)
constexpr int NTN = BN / 16;            // MFMA tiles along the rows
constexpr int NTM = 2;                  // MFMA tiles along the tokens, per wave
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int WS_BYTES = BN * 64 * 2;   // one dequantized-weight buffer (bf16, operand order)
constexpr int kWTasks = BN * 4;         // 16-code quarters of weights per group (576)
constexpr int kWPer = (kWTasks + kThreads - 1) / kThreads;  // 2 (the second: wave 0 only)
constexpr uint32_t kOutside = 0x80000000u;  // buffer offset that reads as zero

// bf16 bit patterns of v = u - 4 for four codes u (one per byte), as the pairs
// [c0 | c1 << 16] and [c2 | c3 << 16].  bf16(v) for v = -4..3 is c080 c040 c000
// bf80 0000 3f80 4000 4040: one table gives the high bytes, one the low bytes.
__device__ __forceinline__ void to_bf16_pairs(uint32_t W4, uint32_t& d0, uint32_t& d1) {
    const uint32_t hi = __builtin_amdgcn_perm(0x40403F00u, 0xBFC0C0C0u, W4);
    const uint32_t lo = __builtin_amdgcn_perm(0x40008000u, 0x80004080u, W4);
    d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// One 16-code quarter: low-plane word L (code 4b+i at bits 8b+2i) and its 16
// high bits h16 (code j at bit j) -> codes 0..7 and 8..15 as bf16x8 (natural
// order, 4 dwords each).
__device__ __forceinline__ void dequant_quarter(uint32_t L, uint32_t h16, u32x4_t& lo8,
                                                u32x4_t& hi8) {
    uint32_t sp = (h16 | (h16 << 8)) & 0x00FF00FFu;
    sp = ((sp | (sp << 4)) & 0x0F0F0F0Fu) << 2;  // code 4b+i's high bit at bit 2+i of byte b
    const uint32_t u0 = (L & 0x03030303u) | (sp & 0x04040404u);
    const uint32_t u1 = ((L >> 2) & 0x03030303u) | ((sp >> 1) & 0x04040404u);
    const uint32_t u2 = ((L >> 4) & 0x03030303u) | ((sp >> 2) & 0x04040404u);
    const uint32_t u3 = ((L >> 6) & 0x03030303u) | ((sp >> 3) & 0x04040404u);
    // byte b of u_i is code 4b+i; regroup into code quads in natural order
    const uint32_t a0 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);  // codes 0 1 4 5
    const uint32_t a1 = __builtin_amdgcn_perm(u1, u0, 0x07030602u);  // codes 8 9 12 13
    const uint32_t b0 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);  // codes 2 3 6 7
    const uint32_t b1 = __builtin_amdgcn_perm(u3, u2, 0x07030602u);  // codes 10 11 14 15
    uint32_t p01, p45, p89, p1213, p23, p67, p1011, p1415;
    to_bf16_pairs(a0, p01, p45);
    to_bf16_pairs(a1, p89, p1213);
    to_bf16_pairs(b0, p23, p67);
    to_bf16_pairs(b1, p1011, p1415);
    lo8 = u32x4_t{p01, p23, p45, p67};
    hi8 = u32x4_t{p89, p1011, p1213, p1415};
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_i3_mfma_kernel(
    const uint8_t* __restrict__ packed, const float* __restrict__ scales, int64_t O, int32_t I,
    int32_t G, const uint16_t* __restrict__ X, int32_t B, float* __restrict__ Y, int32_t ntok,
    int32_t nb) {
    __shared__ __attribute__((aligned(16))) uint8_t ws[2][WS_BYTES];
    __shared__ float ss[2][BN];
    __shared__ __attribute__((aligned(16))) uint8_t raw[2][kThreads * 8];  // rows 0..BN-1: 24 B each
    __shared__ float rawsc[2][kThreads];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h4 = lane >> 4;  // which 8-element slice of an MFMA operand
    const int l16 = lane & 15;
    // Consecutive block ids run on different XCDs (8 of them, each with its
    // own L2): the ids are remapped so that the token blocks of one row block
    // run on one XCD and share its weight lines in that L2.
    int32_t lin = blockIdx.x;
    if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);
    const int64_t n0 = (int64_t)(lin / ntok) * BN;
    const int32_t m0 = (lin % ntok) * BM;

    // ---- activations: buffer over this launch's X, offsets per A slice
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X), (short)0, (int)((int64_t)B * I * 2), 0x00020000);
    uint32_t xoff[NTM][2];  // byte offset of slice (mt, ks) in group 0, or kOutside
#pragma unroll
    for (int mt = 0; mt < NTM; ++mt) {
        const int32_t t = m0 + wave * (16 * NTM) + mt * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            xoff[mt][ks] = t < B ? (uint32_t)(((int64_t)t * I + 32 * ks + 8 * h4) * 2) : kOutside;
    }
    const bool ragged = (I % kGroup) != 0;

    // A slices of group g: 8 registers quads, loaded as raw bf16 bits
    struct ALoad {
        u32x4_t v[NTM][2];
    };
    auto load_a = [&](int32_t g, ALoad& a) {
        uint32_t off[NTM][2];
#pragma unroll
        for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) off[mt][ks] = xoff[mt][ks] + (uint32_t)g * 128u;
        if (ragged && g == G - 1) {  // slices past the row read zeros
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bool inside = g * kGroup + 32 * ks + 8 * h4 < I;
#pragma unroll
                for (int mt = 0; mt < NTM; ++mt)
                    if (!inside) off[mt][ks] = kOutside;
            }
        }
#pragma unroll
        for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if constexpr (VEC) {
                    a.v[mt][ks] = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, off[mt][ks], 0, 0));
                } else {
                    // rows not 16-byte aligned: element loads, each bounded by the row
                    uint32_t w[8];
                    const int32_t k0 = g * kGroup + 32 * ks + 8 * h4;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t oe = (k0 + e < I && off[mt][ks] != kOutside)
                                                ? off[mt][ks] + 2 * e
                                                : kOutside;
                        w[e] = __builtin_amdgcn_raw_buffer_load_b16(xr, oe, 0, 0);
                    }
                    a.v[mt][ks] = u32x4_t{w[0] | (w[1] << 16), w[2] | (w[3] << 16),
                                          w[4] | (w[5] << 16), w[6] | (w[7] << 16)};
                }
            }
    };

    // ---- weights.  Each group's 144 packed rows (24 bytes each) arrive with
    // coalesced 8-byte loads, three consecutive lanes per row, and one f32
    // scale per row; they are parked in a raw LDS slot and dequantized from
    // there by quarter tasks (row, q).  Threads past the tile load a valid
    // row and write to the slot's unused tail, so nothing branches.
    const int rn = min(tid / 3, BN - 1);
    const int64_t wr_row = min<int64_t>(n0 + rn, O - 1);  // rows past O: discarded
    const uint8_t* wptr = packed + wr_row * G * kGroupBytes + 8 * (tid % 3);
    const int64_t sc_row = min<int64_t>(n0 + min(tid, BN - 1), O - 1);
    const float* sptr = scales + sc_row * G;
    struct RawLoad {
        u32x2_t w;
        float s;
    };
    auto load_raw = [&](int32_t g, RawLoad& rl) {
        rl.w = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2_t*>(wptr + (int64_t)g * kGroupBytes));
        rl.s = sptr[g];
    };
    auto write_raw = [&](int slot, const RawLoad& rl) {
        reinterpret_cast<u32x2_t*>(raw[slot])[tid] = rl.w;
        rawsc[slot][tid] = rl.s;
    };
    // dequantize task i from raw slot into LDS buffer buf.  The 64 tasks of
    // chunk c = task / 64 are the quarters q = (task % 64) / 16 of the rows
    // n = 16 c + task % 16 (row tile c).  Codes 16q..16q+7 and 16q+8..16q+15
    // are the operand slices h4 = 2 (q & 1) and 2 (q & 1) + 1 of step
    // ks = q / 2; the four lanes of a row all write its scale.
    auto store_task = [&](int buf, int slot, int i) {
        const int task = tid + kThreads * i;
        const int c = task >> 6, q = (task >> 4) & 3, r16 = task & 15;
        const int n = 16 * c + r16;
        const uint32_t* rw = reinterpret_cast<const uint32_t*>(raw[slot]) + 6 * n;
        const uint32_t lo = rw[q], hw = rw[4 + (q >> 1)];
        u32x4_t lo8, hi8;
        dequant_quarter(lo, (hw >> (16 * (q & 1))) & 0xFFFFu, lo8, hi8);
        u32x4_t* r = reinterpret_cast<u32x4_t*>(ws[buf]) + (2 * c + (q >> 1)) * 64 +
                     32 * (q & 1) + r16;
        r[0] = lo8;
        r[16] = hi8;
        ss[buf][n] = rawsc[slot][n];
    };
    static_assert(kWPer == 2 && kThreads <= kWTasks && kWTasks - kThreads <= 64,
                  "task split: one task per thread plus a remainder for wave 0");
    static_assert(3 * BN <= kThreads && BN <= kThreads, "one raw piece and scale per thread");

    f32x4_t acc[NTM][NTN];
#pragma unroll
    for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One group: MFMAs and scale accumulation from A registers and LDS
    // buffer cb, then the dequantization of the next group's first task into
    // buffer 1-cb.  Row tile nt's B operands are read from LDS two tiles
    // ahead; the scale FMAs of tile nt-1 follow the MFMAs of tile nt, and the
    // scheduling groups at the end ask for three other vector ops after
    // every MFMA, so the FMAs and the dequantization fill the matrix core's
    // shadow.
    auto step = [&](int cb, const ALoad& a) {
        const u32x4_t* wb = reinterpret_cast<const u32x4_t*>(ws[cb]) + lane;
        const float* sb = &ss[cb][l16];
        bf16x8_t aop[NTM][2];
#pragma unroll
        for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) aop[mt][ks] = __builtin_bit_cast(bf16x8_t, a.v[mt][ks]);
        auto read_b = [&](int nt, bf16x8_t (&bb)[2]) {
            bb[0] = __builtin_bit_cast(bf16x8_t, wb[(2 * nt) * 64]);
            bb[1] = __builtin_bit_cast(bf16x8_t, wb[(2 * nt + 1) * 64]);
        };
        float sc[NTN];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) sc[nt] = sb[nt * 16];
        bf16x8_t bring[3][2];
        read_b(0, bring[0]);
        read_b(1, bring[1]);
        f32x4_t part[2][NTM];
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) {
            if (nt + 2 < NTN) read_b(nt + 2, bring[(nt + 2) % 3]);
            const bf16x8_t(&bb)[2] = bring[nt % 3];
#pragma unroll
            for (int mt = 0; mt < NTM; ++mt)
                part[nt & 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    aop[mt][0], bb[0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int mt = 0; mt < NTM; ++mt)
                part[nt & 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    aop[mt][1], bb[1], part[nt & 1][mt], 0, 0, 0);
            if (nt > 0) {
#pragma unroll
                for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[mt][nt - 1][r] = __builtin_fmaf(sc[nt - 1], part[(nt - 1) & 1][mt][r],
                                                            acc[mt][nt - 1][r]);
            }
        }
#pragma unroll
        for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[mt][NTN - 1][r] = __builtin_fmaf(sc[NTN - 1], part[(NTN - 1) & 1][mt][r],
                                                     acc[mt][NTN - 1][r]);
        store_task(1 - cb, 1 - cb, 0);
        // 0x8: MFMA, 0x2: other vector ALU
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int m = 0; m < 2 * NTM; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x2, 3, 0);
            }
    };

    // Software pipeline.  Step k: the A slices of group k are in registers
    // and its weights in LDS buffer k&1; the raw weights of group k+1 wait in
    // raw slot (k+1)&1 and those of k+2 in registers.  It issues the loads of
    // A(k+kAhead) and of the raw weights of k+3, multiplies group k,
    // dequantizes k+1 into the other buffer and parks the raw weights of k+2
    // in slot k&1.  With 16-byte activation loads the A slices come from a
    // ring of three, two groups in flight (a load waits for the loads issued
    // before it, raw weights from HBM among them): 3 % faster at the prefill
    // shape than one group ahead.  The element-load path keeps one group in
    // flight, which fits its registers.  The loop is unrolled so that every
    // ring slot is a fixed register set, and its body is straight-line
    // (prefetches past the last group re-read group G-1 and land where nobody
    // reads): loads issued under conditions keep the compiler from telling
    // which are still in flight.
    constexpr int kAhead = VEC ? 2 : 1;
    ALoad a0, a1, a2;
    RawLoad ra, rb;
    const int32_t glast = G - 1;
    load_a(0, a0);
    if constexpr (kAhead == 2) load_a(min(1, glast), a1);
    load_raw(0, ra);
    load_raw(min(1, glast), rb);
    write_raw(0, ra);
    write_raw(1, rb);
    lds_barrier();
    store_task(0, 0, 0);
    if (wave == 0) store_task(0, 0, 1);
    load_raw(min(2, glast), ra);
    lds_barrier();
    // group g (LDS buffer cb = g & 1) with A slices acur; A(g+kAhead) into
    // anext, raw(g+3) into rload; rwrite holds raw(g+2).  True after the
    // last group.
    auto group = [&](int32_t g, int cb, const ALoad& acur, ALoad& anext, RawLoad& rload,
                     const RawLoad& rwrite) {
        load_a(min(g + kAhead, glast), anext);
        load_raw(min(g + 3, glast), rload);
        step(cb, acur);
        if (wave == 0) store_task(1 - cb, 1 - cb, 1);
        write_raw(cb, rwrite);
        lds_barrier();
        return g + 1 >= G;
    };
    if constexpr (kAhead == 2) {
        for (int32_t g = 0;; g += 6) {
            if (group(g + 0, 0, a0, a2, rb, ra)) break;
            if (group(g + 1, 1, a1, a0, ra, rb)) break;
            if (group(g + 2, 0, a2, a1, rb, ra)) break;
            if (group(g + 3, 1, a0, a2, ra, rb)) break;
            if (group(g + 4, 0, a1, a0, rb, ra)) break;
            if (group(g + 5, 1, a2, a1, ra, rb)) break;
        }
    } else {
        for (int32_t g = 0;; g += 2) {
            if (group(g + 0, 0, a0, a1, rb, ra)) break;
            if (group(g + 1, 1, a1, a0, ra, rb)) break;
        }
    }

    // C layout of a 16x16 tile: register r of lane l holds token row
    // 4*(l/16) + r and output column l%16.
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt) {
        const int64_t o = n0 + nt * 16 + l16;
        if (o >= O) continue;
#pragma unroll
        for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t t = m0 + wave * (16 * NTM) + mt * 16 + 4 * h4 + r;
                if (t < B) Y[(int64_t)t * O + o] = acc[mt][nt][r];
            }
    }
}

}  // namespace

hipError_t launch_gemm_mfma(const uint8_t* packed, const float* scales, int64_t O,
                            int64_t I, const uint16_t* X, int64_t B, float* Y,
                            hipStream_t s) {
    const int64_t G = (I + kGroup - 1) / kGroup;
    // The activation buffer of one launch spans at most 2^31 - 1 bytes (its
    // out-of-range offset is 2^31), so long batches go in token slabs.
    const int64_t slab = ((0x7FFFFFFFLL / (I * 2)) / BM) * BM;
    if (slab < BM || G > 0x7FFFFFFF) return hipErrorInvalidValue;
    const bool vec = (I % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    for (int64_t t0 = 0; t0 < B; t0 += slab) {
        const int64_t bt = min(slab, B - t0);
        const int32_t ntok = (int32_t)((bt + BM - 1) / BM);
        const int64_t nb = ((O + BN - 1) / BN) * ntok;
        if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
        const dim3 grid((unsigned)nb);
        if (vec)
            hipLaunchKernelGGL((gemm_i3_mfma_kernel<true>), grid, dim3(kThreads), 0, s, packed,
                               scales, O, (int32_t)I, (int32_t)G, X + t0 * I, (int32_t)bt,
                               Y + t0 * O, ntok, (int32_t)nb);
        else
            hipLaunchKernelGGL((gemm_i3_mfma_kernel<false>), grid, dim3(kThreads), 0, s, packed,
                               scales, O, (int32_t)I, (int32_t)G, X + t0 * I, (int32_t)bt,
                               Y + t0 * O, ntok, (int32_t)nb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qt
