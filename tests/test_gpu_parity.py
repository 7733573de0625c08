"""HIP path against the CPU oracle, element by element, through the C ABI.

Bit-exact: codes, scales, chosen grid indices, packed bytes.  Floating point:
the exact-f32 multiply paths within 1e-5 and the bf16 MFMA path within 2e-3 of
sum_i |w_oi x_i| (componentwise against the fp64 dequantize-then-multiply).
"""
import numpy as np
import pytest
import torch

import dequant_matmul_int3_amd as qt
import oracle
import workloads
from tests.gpu_util import bits, dev, dev_bf16, host, say
from tests.parity import componentwise_err, np_decode_planes

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_MFMA = 2e-3


def tol_mfma_exact_codes(I):
    """The MFMA path's own bound: codes and bf16 inputs multiply exactly, each
    64-input group is summed in f32 (at most 63 roundings), scaled once and
    added to an f32 total over G groups (G - 1 roundings): to first order
    (64 + G + 1) * 2^-24 of sum |w x|.  The contract's 2e-3 is the outer bar;
    this one catches a regression of the kernel's own arithmetic."""
    return (64 + (I + 63) // 64 + 2) * 2.0 ** -24


def gpu_quantize_pack(W, d=None, n_grid=0, lo=0.5, hi=1.0):
    Wd = dev(W)
    dd = None if d is None else dev(d)
    s, c, k = qt.qt_quantize_g64(Wd, dd, n_grid, lo, hi)
    p = qt.qt_pack_i3(c)
    return host(s), host(c), host(k), host(p), (p, s)


def check_quantize(W, d=None, n_grid=0, lo=0.5, hi=1.0):
    O, I = W.shape
    say(f"quantize+pack O={O} I={I} n_grid={n_grid}")
    s, c, k, p, devbufs = gpu_quantize_pack(W, d, n_grid, lo, hi)
    so, co, ko = oracle.quantize_g64(W, d, n_grid, lo, hi)
    po = oracle.pack_i3(co)
    assert np.array_equal(bits(s), bits(so)), "scales differ"
    assert np.array_equal(c, co), "codes differ"
    assert np.array_equal(k, ko), "grid indices differ"
    assert np.array_equal(p, po), "packed bytes differ"
    return so, co, po, devbufs


# ---------------------------------------------------------------- quantize / pack
def test_tiny_quantize_pack_matvec_and_outlier_rows():
    W, x, rows = workloads.tiny()
    O, I = W.shape
    so, co, po, (pd, sd) = check_quantize(W)
    say("matvec tiny")
    y = host(qt.qt_matvec_i3(pd, sd, O, I, dev(x)))
    yr, ar = oracle.matvec_f64(po, so, O, I, x)
    assert componentwise_err(y, yr, ar) <= TOL_F32
    # outlier rows: the GPU-produced int3-g64 reconstruction beats per-row int4
    what = np_decode_planes(host(pd), O, I).astype(np.float64) * np.repeat(
        host(sd).astype(np.float64), 64, axis=1)[:, :I]
    r3 = what[rows] - W[rows]
    r4 = oracle.rowint_recon(W, 4)[rows] - W[rows]
    assert np.sqrt(np.mean(r3 ** 2)) < np.sqrt(np.mean(r4 ** 2))


@pytest.mark.parametrize("tail", [False, True])
def test_decode_quantize_pack_matvec(tail):
    W, x = workloads.decode(tail)
    O, I = W.shape
    so, co, po, (pd, sd) = check_quantize(W)
    say(f"matvec decode I={I}")
    y1 = qt.qt_matvec_i3(pd, sd, O, I, dev(x))
    y2 = qt.qt_matvec_i3(pd, sd, O, I, dev(x))
    y1, y2 = host(y1), host(y2)
    assert np.array_equal(bits(y1), bits(y2)), "matvec is not deterministic"
    yr, ar = oracle.matvec_f64(po, so, O, I, x)
    err = componentwise_err(y1, yr, ar)
    say(f"  componentwise err {err:.3e}")
    assert err <= TOL_F32


SHAPES = [(1, 1), (1, 64), (3, 65), (17, 100), (33, 129), (5, 7200), (300, 64), (7, 1000),
          (129, 640), (2, 4097)]


@pytest.mark.parametrize("O,I", SHAPES)
def test_ragged_quantize_pack_matvec(O, I):
    W = workloads.generic_weights(O, I, seed=O * 7919 + I)
    so, co, po, (pd, sd) = check_quantize(W)
    x = workloads.generic_vector(I, seed=I)
    say(f"matvec ragged O={O} I={I}")
    y = host(qt.qt_matvec_i3(pd, sd, O, I, dev(x)))
    yr, ar = oracle.matvec_f64(po, so, O, I, x)
    assert componentwise_err(y, yr, ar) <= TOL_F32


@pytest.mark.parametrize("n_grid,lo,hi", [(64, 0.5, 1.0), (2, 0.5, 1.0), (256, 0.3, 1.2),
                                          (17, 0.75, 0.75)])
@pytest.mark.parametrize("weighted", [False, True])
def test_search_bit_exact(n_grid, lo, hi, weighted):
    O, I = 64, 1000
    W = workloads.generic_weights(O, I, seed=n_grid)
    W[3, :64] = 0.0  # an all-zero group
    d = None
    if weighted:
        d = np.exp(workloads.generic_vector(I, seed=5)).astype(np.float32)
        d[7] = 0.0
    check_quantize(W, d, n_grid, lo, hi)


def test_search_summation_order_group():
    # the group of tests/golden/search_order.txt, on which a left-to-right sum
    # of the objective picks another scale than the halving order; placed in
    # several rows and in both the first and a later group of a row
    from tests.test_oracle import read_search_order_fixture
    w, d, n, lo, hi, k, scale, codes = read_search_order_fixture()
    W = np.zeros((8, 192), np.float32)
    dd = np.ones(192, np.float32)
    for o in range(8):
        g = o % 3
        W[o, 64 * g:64 * g + 64] = w
    for g in range(3):
        dd[64 * g:64 * g + 64] = d
    so, co, _, _ = check_quantize(W, dd, n, lo, hi)
    for o in range(8):
        g = o % 3
        assert so[o, g] == scale and np.array_equal(co[o, 64 * g:64 * g + 64], codes)


def check_signed(W, d, n1, n2, lo=0.5, hi=1.0):
    O, I = W.shape
    say(f"signed search O={O} I={I} n1={n1} n2={n2} weighted={d is not None}")
    s, c = qt.qt_quantize_g64_signed(dev(W), None if d is None else dev(d), n1, n2, lo, hi)
    s, c = host(s), host(c)
    so, co = oracle.quantize_g64_signed(W, d, n1, n2, lo, hi)
    assert np.array_equal(bits(s), bits(so)), "scales differ"
    assert np.array_equal(c, co), "codes differ"
    # the packed planes of negative-scale groups multiply like any other
    p = host(qt.qt_pack_i3(dev(c)))
    assert np.array_equal(p, oracle.pack_i3(co))
    return so, co


@pytest.mark.parametrize("n1,n2,lo,hi", [(64, 32, 0.5, 1.0), (64, 0, 0.5, 1.0),
                                         (16, 8, 0.3, 1.2), (2, 2, 0.75, 0.75)])
@pytest.mark.parametrize("weighted", [False, True])
def test_signed_search_bit_exact(n1, n2, lo, hi, weighted):
    O, I = 70, 1000
    W = workloads.generic_weights(O, I, seed=100 + n1 + n2)
    W[5, 64:128] = 0.0  # an all-zero group
    d = None
    if weighted:
        d = np.exp(workloads.generic_vector(I, seed=6)).astype(np.float32)
        d[9] = 0.0
    so, co = check_signed(W, d, n1, n2, lo, hi)
    # some groups really choose a negative scale
    assert np.any(so < 0) and np.any(so > 0)


def test_signed_search_special_groups_and_matvec():
    O, I = 6, 192
    W = np.zeros((O, I), np.float32)
    W[0, 0] = 4.0                     # best scale -1: 4 on code -4 exactly
    W[1, :] = -0.5                    # equal magnitudes of one sign
    W[2] = np.tile(np.array([1.0, -1.0, 0.5, -0.5], np.float32), I // 4)
    W[3, 7] = 3.0e-39                 # subnormal group maximum
    W[4] = workloads.generic_weights(1, I, seed=8)[0] * np.float32(1e30)
    W[5] = workloads.generic_weights(1, I, seed=9)[0]
    so, co = check_signed(W, None, 64, 32)
    assert so[0, 0] == np.float32(-1.0) and co[0, 0] == -4
    # a matvec over signed scales against the f64 reference
    po = oracle.pack_i3(co)
    x = workloads.generic_vector(I, seed=10)
    y = host(qt.qt_matvec_i3(dev(po), dev(so), O, I, dev(x)))
    yr, ar = oracle.matvec_f64(po, so, O, I, x)
    assert componentwise_err(y, yr, ar) <= TOL_F32


def test_search_ties_and_special_groups():
    # groups built so that many candidates tie exactly (equal magnitudes on a
    # power-of-two grid); the lowest k must win on both sides
    O, I = 8, 256
    W = np.zeros((O, I), np.float32)
    W[0] = 0.5
    W[1, ::2] = -0.25
    W[2] = np.tile(np.array([1.0, -1.0, 0.5, -0.5], np.float32), I // 4)
    W[3, 5] = 3.0e-39  # a subnormal group maximum
    W[4] = workloads.generic_weights(1, I, seed=3)[0] * np.float32(1e30)
    W[5, 100] = -1.0
    W[6] = np.float32(1e-30)
    W[7] = workloads.generic_weights(1, I, seed=4)[0]
    check_quantize(W, None, 64, 0.5, 1.0)
    check_quantize(W, np.full(I, 2.0, np.float32), 64, 0.5, 1.0)


@pytest.mark.parametrize("O,I", [(5, 64), (9, 100), (64, 7200), (3, 1)])
def test_pack_random_codes(O, I):
    rng = workloads.rng_for("generic", 31, O, I)
    codes = rng.integers(-4, 4, size=(O, I)).astype(np.int8)
    say(f"pack O={O} I={I}")
    p = host(qt.qt_pack_i3(dev(codes)))
    assert np.array_equal(p, oracle.pack_i3(codes))


# ---------------------------------------------------------------- matvec properties
@pytest.mark.parametrize("O,I", [(4104, 7168), (6000, 1000), (5000, 130)])
def test_matvec_many_row_tiles(O, I):
    # more than 512 tiles of 8 rows: the decode kernel's looping form (each
    # block takes several tiles, the next ones in flight), with a partly
    # used last tile and, for I = 130, a short tail group
    W = workloads.generic_weights(O, I, seed=O + I)
    so, co, po, (pd, sd) = check_quantize(W)
    x = workloads.generic_vector(I, seed=7)
    say(f"matvec many tiles O={O} I={I}")
    y = host(qt.qt_matvec_i3(pd, sd, O, I, dev(x)))
    yr, ar = oracle.matvec_f64(po, so, O, I, x)
    assert componentwise_err(y, yr, ar) <= TOL_F32
    y2 = host(qt.qt_matvec_i3(pd, sd, O, I, dev(x)))
    assert np.array_equal(bits(y), bits(y2)), "matvec is not deterministic"


def test_matvec_one_hot_is_exact():
    O, I = 64, 300
    W = workloads.generic_weights(O, I, seed=12)
    so, co, po, (pd, sd) = check_quantize(W)
    for i in (0, 63, 64, 200, 299):
        x = np.zeros(I, np.float32)
        x[i] = 1.0
        say(f"one-hot i={i}")
        y = host(qt.qt_matvec_i3(pd, sd, O, I, dev(x)))
        assert np.array_equal(y, so[:, i // 64] * co[:, i].astype(np.float32))


def test_matvec_zero_weights():
    O, I = 16, 200
    W = np.zeros((O, I), np.float32)
    so, co, po, (pd, sd) = check_quantize(W)
    y = host(qt.qt_matvec_i3(pd, sd, O, I, dev(workloads.generic_vector(I))))
    assert np.all(y == 0)


# ---------------------------------------------------------------- batched multiply
def _packed_for(O, I, seed):
    W = workloads.generic_weights(O, I, seed=seed)
    so, co, _ = oracle.quantize_g64(W)
    po = oracle.pack_i3(co)
    return so, po


def _matmul_ref(po, so, O, I, X):
    B = X.shape[0]
    t = np.repeat(np.arange(B), O)
    o = np.tile(np.arange(O), B)
    y, a = oracle.matmul_f64_sampled(po, so, O, I, X, t, o)
    return y.reshape(B, O), a.reshape(B, O)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9, 15, 16, 17, 40])
def test_matmul_f32_exact_path(B):
    O, I = 70, 650
    so, po = _packed_for(O, I, seed=B)
    X = workloads.generic_matrix(B, I, seed=B)
    say(f"matmul f32 B={B}")
    Y = host(qt.qt_matmul_i3(dev(po), dev(so), O, I, dev(X)))
    yr, ar = _matmul_ref(po, so, O, I, X)
    assert componentwise_err(Y, yr, ar) <= TOL_F32


@pytest.mark.parametrize("B", [1, 2, 4, 6, 12])
def test_matmul_f32_exact_path_several_chunks(B):
    # 141 groups: more than one staged chunk of inputs for every tile width,
    # 16-byte input rows, and a last block of rows that is only partly used
    O, I = 37, 9000
    so, po = _packed_for(O, I, seed=300 + B)
    X = workloads.generic_matrix(B, I, seed=310 + B)
    say(f"matmul f32 chunks B={B}")
    Y = host(qt.qt_matmul_i3(dev(po), dev(so), O, I, dev(X)))
    yr, ar = _matmul_ref(po, so, O, I, X)
    assert componentwise_err(Y, yr, ar) <= TOL_F32


@pytest.mark.parametrize("B", [1, 2, 4, 7, 15])
def test_matmul_bf16_small_batch_exact_path(B):
    O, I = 50, 300
    so, po = _packed_for(O, I, seed=100 + B)
    Xb = workloads.bf16_bits_rne(workloads.generic_matrix(B, I, seed=B))
    say(f"matmul bf16 small B={B}")
    Y = host(qt.qt_matmul_i3(dev(po), dev(so), O, I, dev_bf16(Xb)))
    yr, ar = _matmul_ref(po, so, O, I, workloads.bf16_bits_to_f32(Xb))
    assert componentwise_err(Y, yr, ar) <= TOL_F32


# The 16-byte-load path runs its group loop in rounds of six; G = 1, 2, 3,
# 5, 6, 7, 10, 16 and 112 end a round at every position.
@pytest.mark.parametrize("B,O,I", [(16, 128, 64), (17, 200, 300), (130, 129, 640),
                                   (300, 64, 1000), (256, 256, 7168), (33, 40, 68),
                                   (20, 31, 5), (24, 48, 128), (40, 96, 192),
                                   (260, 150, 320), (64, 80, 384), (18, 144, 448)])
def test_matmul_bf16_mfma_path(B, O, I):
    so, po = _packed_for(O, I, seed=B + O + I)
    Xb = workloads.bf16_bits_rne(workloads.generic_matrix(B, I, seed=B + I))
    say(f"matmul bf16 mfma B={B} O={O} I={I}")
    Yd1 = qt.qt_matmul_i3(dev(po), dev(so), O, I, dev_bf16(Xb))
    Yd2 = qt.qt_matmul_i3(dev(po), dev(so), O, I, dev_bf16(Xb))
    Y, Y2 = host(Yd1), host(Yd2)
    assert np.array_equal(bits(Y), bits(Y2)), "matmul is not deterministic"
    yr, ar = _matmul_ref(po, so, O, I, workloads.bf16_bits_to_f32(Xb))
    err = componentwise_err(Y, yr, ar)
    say(f"  componentwise err {err:.3e}")
    assert err <= TOL_MFMA
    assert err <= tol_mfma_exact_codes(I)


def test_matmul_b1_equals_matvec():
    O, I = 100, 777
    so, po = _packed_for(O, I, seed=2)
    x = workloads.generic_vector(I, seed=3)
    y1 = host(qt.qt_matvec_i3(dev(po), dev(so), O, I, dev(x)))
    y2 = host(qt.qt_matmul_i3(dev(po), dev(so), O, I, dev(x[None, :])))
    assert np.array_equal(bits(y1), bits(y2[0]))


# ---------------------------------------------------------------- pointer alignment
def _at_offset(t, off):
    """A device copy of t whose first byte lies `off` bytes past a 256-byte
    boundary (torch allocations start on such a boundary)."""
    esz = t.element_size()
    assert off % esz == 0
    n = t.numel()
    buf = torch.empty(n + 256 // esz, dtype=t.dtype, device=t.device)
    k = ((off - buf.data_ptr()) % 256) // esz
    v = buf[k:k + n]
    v.copy_(t.reshape(-1))
    assert v.data_ptr() % 256 == off
    return v.view(t.shape)


@pytest.mark.parametrize("poff", [4, 12])
def test_unaligned_packed_and_bf16_inputs(poff):
    # packed at 4 (not 8) and 12 (not 16) bytes, bf16 X at 2 bytes: every
    # int3 entry point gives the bytes / bits of the aligned call
    O, I = 70, 650  # G = 11: 24-byte groups alternate between 8- and 16-byte offsets
    W = workloads.generic_weights(O, I, seed=900 + poff)
    so, co, _ = oracle.quantize_g64(W)
    po = oracle.pack_i3(co)
    say(f"unaligned packed +{poff}: pack")
    pko = _at_offset(torch.zeros(po.size, dtype=torch.uint8, device="cuda:0"), poff)
    qt.qt_pack_i3(dev(co), pko)
    assert np.array_equal(host(pko), po)
    pk, sc = dev(po), dev(so)
    say(f"unaligned packed +{poff}: matvec")
    x = dev(workloads.generic_vector(I, seed=5))
    assert np.array_equal(bits(host(qt.qt_matvec_i3(pko, sc, O, I, x))),
                          bits(host(qt.qt_matvec_i3(pk, sc, O, I, x))))
    for B in (7, 20):  # exact path, MFMA path
        say(f"unaligned packed +{poff}, bf16 X +2: matmul B={B}")
        Xb = dev_bf16(workloads.bf16_bits_rne(workloads.generic_matrix(B, I, seed=B)))
        Xo = _at_offset(Xb, 2)
        ref = host(qt.qt_matmul_i3(pk, sc, O, I, Xb))
        for pp, xx in ((pko, Xb), (pk, Xo), (pko, Xo)):
            assert np.array_equal(bits(host(qt.qt_matmul_i3(pp, sc, O, I, xx))), bits(ref))
        yr, ar = _matmul_ref(po, so, O, I, workloads.bf16_bits_to_f32(host(Xb)))
        assert componentwise_err(ref, yr, ar) <= (TOL_F32 if B < 16 else tol_mfma_exact_codes(I))
    say(f"unaligned packed +{poff}: grouped")
    E, T = 3, 5
    tok = np.array([0, 2, 4, 1, 3, 4], np.int32)
    offs = np.array([0, 2, 4, 6], np.int32)
    pe = np.concatenate([po] * E)
    se = np.concatenate([so] * E)
    X = workloads.generic_matrix(T, I, seed=31)
    pke = dev(pe)
    pkeo = _at_offset(pke, poff)
    args = (dev(se), E, O, I, dev(X), dev(offs), tok.size)
    y1 = host(qt.qt_matvec_i3_grouped(pke, *args, pair_row=dev(tok)))
    y2 = host(qt.qt_matvec_i3_grouped(pkeo, *args, pair_row=dev(tok)))
    assert np.array_equal(bits(y1), bits(y2))


# ---------------------------------------------------------------- grouped (MoE)
def _grouped_case(E, O, I, T, topk, seed):
    rng = workloads.rng_for("generic", 500 + seed, E, O, I)
    logits = rng.random((T, E))
    top = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    tok, exp, offs = workloads.route_pairs(top, E)
    Ws = [workloads.generic_weights(O, I, seed=1000 * seed + e) for e in range(E)]
    q = [oracle.quantize_g64(w) for w in Ws]
    so = np.stack([a[0] for a in q])
    po = np.stack([oracle.pack_i3(a[1]) for a in q])
    X = workloads.generic_matrix(T, I, seed=seed)
    return tok, exp, offs, so, po, X


@pytest.mark.parametrize("E,O,I,T,topk", [(4, 40, 300, 6, 2), (16, 64, 1000, 32, 8),
                                          (3, 100, 64, 40, 3), (8, 33, 7200, 5, 1),
                                          (5, 130, 450, 12, 3), (3, 70, 130, 9, 2)])
def test_grouped_matvec(E, O, I, T, topk):
    tok, exp, offs, so, po, X = _grouped_case(E, O, I, T, topk, seed=E + T)
    P = tok.size
    say(f"grouped E={E} O={O} I={I} P={P}")
    Y = host(qt.qt_matvec_i3_grouped(dev(po), dev(so), E, O, I, dev(X), dev(offs), P,
                                     pair_row=dev(tok)))
    for p in range(P):
        e, t = exp[p], tok[p]
        yr, ar = oracle.matvec_f64(po[e], so[e], O, I, X[t])
        assert componentwise_err(Y[p], yr, ar) <= TOL_F32, (p, e, t)
    # rows taken by pair index (no pair_row): the down-projection form
    H = workloads.generic_matrix(P, I, seed=77)
    Y2 = host(qt.qt_matvec_i3_grouped(dev(po), dev(so), E, O, I, dev(H), dev(offs), P))
    for p in range(P):
        yr, ar = oracle.matvec_f64(po[exp[p]], so[exp[p]], O, I, H[p])
        assert componentwise_err(Y2[p], yr, ar) <= TOL_F32


def test_grouped_empty_experts_and_one_pair():
    E, O, I = 6, 20, 130
    tok = np.array([3], np.int32)
    offs = np.array([0, 0, 0, 1, 1, 1, 1], np.int32)
    Ws = [workloads.generic_weights(O, I, seed=e) for e in range(E)]
    q = [oracle.quantize_g64(w) for w in Ws]
    so = np.stack([a[0] for a in q])
    po = np.stack([oracle.pack_i3(a[1]) for a in q])
    X = workloads.generic_matrix(4, I, seed=1)
    Y = host(qt.qt_matvec_i3_grouped(dev(po), dev(so), E, O, I, dev(X), dev(offs), 1,
                                     pair_row=dev(tok)))
    yr, ar = oracle.matvec_f64(po[2], so[2], O, I, X[3])
    assert componentwise_err(Y[0], yr, ar) <= TOL_F32


# ---------------------------------------------------------------- Hessian diagonal
@pytest.mark.parametrize("T,I", [(1, 1), (7, 100), (128, 64), (129, 1000), (1000, 333),
                                 (4096, 2048)])
@pytest.mark.parametrize("xt", ["f32", "bf16"])
def test_hessian_diag(T, I, xt):
    X = workloads.generic_matrix(T, I, seed=T + I) * np.exp(
        workloads.generic_vector(I, seed=9))[None, :].astype(np.float32)
    X = X.astype(np.float32)
    if xt == "bf16":
        Xb = workloads.bf16_bits_rne(X)
        Xh = workloads.bf16_bits_to_f32(Xb)
        Xd = dev_bf16(Xb)
    else:
        Xh, Xd = X, dev(X)
    say(f"hessian T={T} I={I} {xt}")
    d = host(qt.qt_hessian_diag(Xd))
    ref = oracle.hessian_diag(Xh)
    assert np.all(np.abs(d - ref) <= 1e-5 * ref + 1e-30)
    # accumulate: two halves equal one pass
    h = T // 2
    if h > 0:
        dd = qt.qt_hessian_diag(Xd[:h].contiguous())
        qt.qt_hessian_diag(Xd[h:].contiguous(), d=dd, accumulate=True)
        assert np.all(np.abs(host(dd) - ref) <= 1e-5 * ref + 1e-30)


def test_hessian_constant_columns_closed_form():
    T, I = 3000, 256
    X = np.ones((T, I), np.float32)
    d = host(qt.qt_hessian_diag(dev(X)))
    assert np.array_equal(d, np.full(I, float(T), np.float32))


def test_search_quotients_on_and_next_to_half_integers():
    # weights whose quotient w/s falls exactly on a half-integer, or one ulp
    # beside it, for the scale of a chosen candidate: rounding ties and
    # near-ties must be decided exactly as the correctly rounded division does
    rng = workloads.rng_for("generic", 4711)
    fk = np.linspace(0.5, 1.0, 64).astype(np.float32)
    rows = []
    for r in range(48):
        b = np.float32(rng.uniform(0.01, 0.05))
        k = int(rng.integers(0, 64))
        s = np.float32(b * fk[k])
        w = np.empty(64, np.float32)
        w[0] = np.float32(4.0) * b  # the group maximum: base = b exactly
        for j in range(1, 64):
            h = np.float32(int(rng.integers(-4, 4)) + 0.5)
            v = np.float32(h * s)
            step = int(rng.integers(-1, 2))
            w[j] = np.nextafter(v, np.float32(np.inf) if step > 0 else np.float32(-np.inf)) \
                if step else v
        w = np.clip(w, -w[0], w[0])
        rows.append(w)
    W = np.stack(rows).astype(np.float32)
    check_quantize(W, None, 64, 0.5, 1.0)
    check_quantize(W, None, 0)
    d = np.exp(workloads.generic_vector(64, seed=17)).astype(np.float32)
    check_quantize(W, d, 64, 0.5, 1.0)
    # the signed search meets the same quotients with both signs
    check_signed(W, None, 64, 32)
    check_signed(W, d, 64, 0)
