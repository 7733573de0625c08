"""Grouped int4 HIP path against the CPU oracle, through the C ABI.

Bit-exact: codes, scales, chosen grid indices and packed bytes.  The exact-f32
multiply (one vector or a batch) within 1e-5 of sum_i |w_oi x_i| of the fp64
dequantize-then-multiply value.
"""
import numpy as np
import pytest

import dequant_matmul_int3_amd as qt
import oracle
import workloads
from tests.gpu_util import bits, dev, dev_bf16, host, say
from tests.parity import componentwise_err

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


def check_quantize_i4(W, d=None, n_grid=0, lo=0.5, hi=1.0):
    O, I = W.shape
    say(f"int4 quantize+pack O={O} I={I} n_grid={n_grid} weighted={d is not None}")
    sd, cd, kd = qt.qt_quantize_g64_i4(dev(W), None if d is None else dev(d), n_grid, lo, hi)
    pd = qt.qt_pack_i4(cd)
    s, c, k, p = host(sd), host(cd), host(kd), host(pd)
    so, co, ko = oracle.quantize_g64_i4(W, d, n_grid, lo, hi)
    po = oracle.pack_i4(co)
    assert np.array_equal(bits(s), bits(so)), "scales differ"
    assert np.array_equal(c, co), "codes differ"
    assert np.array_equal(k, ko), "grid indices differ"
    assert np.array_equal(p, po), "packed bytes differ"
    return so, co, po, (pd, sd)


def matvec_ref(po, so, O, I, x):
    return oracle.matvec_i4_f64(po, so, O, I, x)


SHAPES = [(1, 1), (1, 64), (3, 65), (17, 100), (33, 129), (5, 7200), (300, 64), (7, 1000),
          (129, 640), (2, 4097)]


@pytest.mark.parametrize("O,I", SHAPES)
def test_i4_ragged_quantize_pack_matvec(O, I):
    W = workloads.generic_weights(O, I, seed=O * 7907 + I)
    so, co, po, (pd, sd) = check_quantize_i4(W)
    x = workloads.generic_vector(I, seed=I + 1)
    say(f"int4 matvec O={O} I={I}")
    y = host(qt.qt_matvec_i4(pd, sd, O, I, dev(x)))
    yr, ar = matvec_ref(po, so, O, I, x)
    assert componentwise_err(y, yr, ar) <= TOL_F32


@pytest.mark.parametrize("tail", [False, True])
def test_i4_decode_quantize_pack_matvec(tail):
    W, x = workloads.decode(tail)
    O, I = W.shape
    so, co, po, (pd, sd) = check_quantize_i4(W)
    say(f"int4 matvec decode I={I}")
    y1 = host(qt.qt_matvec_i4(pd, sd, O, I, dev(x)))
    y2 = host(qt.qt_matvec_i4(pd, sd, O, I, dev(x)))
    assert np.array_equal(bits(y1), bits(y2)), "matvec is not deterministic"
    yr, ar = matvec_ref(po, so, O, I, x)
    err = componentwise_err(y1, yr, ar)
    say(f"  componentwise err {err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("n_grid,lo,hi", [(64, 0.5, 1.0), (2, 0.5, 1.0), (256, 0.3, 1.2),
                                          (17, 0.75, 0.75)])
@pytest.mark.parametrize("weighted", [False, True])
def test_i4_search_bit_exact(n_grid, lo, hi, weighted):
    O, I = 64, 1000
    W = workloads.generic_weights(O, I, seed=n_grid + 3)
    W[3, :64] = 0.0  # an all-zero group
    d = None
    if weighted:
        d = np.exp(workloads.generic_vector(I, seed=6)).astype(np.float32)
        d[7] = 0.0
    check_quantize_i4(W, d, n_grid, lo, hi)


def test_i4_ties_and_special_groups():
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
    check_quantize_i4(W, None, 0)
    check_quantize_i4(W, None, 64, 0.5, 1.0)
    check_quantize_i4(W, np.full(I, 2.0, np.float32), 64, 0.5, 1.0)


def test_i4_quotients_on_and_next_to_half_integers():
    # quotients w/s exactly on a half-integer of [-8, 7], or one ulp beside it,
    # for the scale of a chosen candidate: the reciprocal shortcut must decide
    # them as the correctly rounded division does
    rng = workloads.rng_for("generic", 4712)
    fk = np.linspace(0.5, 1.0, 64).astype(np.float32)
    rows = []
    for _ in range(48):
        b = np.float32(rng.uniform(0.01, 0.05))
        k = int(rng.integers(0, 64))
        s = np.float32(b * fk[k])
        w = np.empty(64, np.float32)
        w[0] = np.float32(8.0) * b  # the group maximum: base = b exactly
        for j in range(1, 64):
            h = np.float32(int(rng.integers(-8, 8)) + 0.5)
            v = np.float32(h * s)
            step = int(rng.integers(-1, 2))
            w[j] = np.nextafter(v, np.float32(np.inf) if step > 0 else np.float32(-np.inf)) \
                if step else v
        w = np.clip(w, -w[0], w[0])
        rows.append(w)
    W = np.stack(rows).astype(np.float32)
    check_quantize_i4(W, None, 64, 0.5, 1.0)
    check_quantize_i4(W, None, 0)
    d = np.exp(workloads.generic_vector(64, seed=18)).astype(np.float32)
    check_quantize_i4(W, d, 64, 0.5, 1.0)


@pytest.mark.parametrize("O,I", [(5, 64), (9, 100), (64, 7200), (3, 1)])
def test_i4_pack_codes_in_and_out_of_range(O, I):
    rng = workloads.rng_for("generic", 37, O, I)
    codes = rng.integers(-8, 8, size=(O, I)).astype(np.int8)
    say(f"int4 pack O={O} I={I}")
    assert np.array_equal(host(qt.qt_pack_i4(dev(codes))), oracle.pack_i4(codes))
    # codes outside [-8, 7] keep the low four bits of v + 8
    wide = rng.integers(-128, 128, size=(O, I)).astype(np.int8)
    assert np.array_equal(host(qt.qt_pack_i4(dev(wide))), oracle.pack_i4(wide))


def test_i4_matvec_one_hot_is_exact():
    O, I = 64, 300
    W = workloads.generic_weights(O, I, seed=13)
    so, co, po, (pd, sd) = check_quantize_i4(W)
    for i in (0, 1, 7, 8, 63, 64, 200, 299):
        x = np.zeros(I, np.float32)
        x[i] = 1.0
        say(f"int4 one-hot i={i}")
        y = host(qt.qt_matvec_i4(pd, sd, O, I, dev(x)))
        assert np.array_equal(y, so[:, i // 64] * co[:, i].astype(np.float32))


def _i4_packed_for(O, I, seed):
    W = workloads.generic_weights(O, I, seed=seed)
    so, co, _ = oracle.quantize_g64_i4(W)
    return so, oracle.pack_i4(co)


def _matmul_ref(po, so, O, I, X):
    ys, zs = zip(*(matvec_ref(po, so, O, I, X[t]) for t in range(X.shape[0])))
    return np.stack(ys), np.stack(zs)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9, 16, 17, 40])
def test_i4_matmul_f32(B):
    O, I = 70, 650
    so, po = _i4_packed_for(O, I, seed=B + 1)
    X = workloads.generic_matrix(B, I, seed=B + 2)
    say(f"int4 matmul f32 B={B}")
    Y = host(qt.qt_matmul_i4(dev(po), dev(so), O, I, dev(X)))
    yr, ar = _matmul_ref(po, so, O, I, X)
    assert componentwise_err(Y, yr, ar) <= TOL_F32


@pytest.mark.parametrize("B", [1, 2, 4, 6, 12])
def test_i4_matmul_f32_several_chunks(B):
    # 141 groups: more than one staged chunk of inputs for every tile width
    O, I = 37, 9000
    so, po = _i4_packed_for(O, I, seed=400 + B)
    X = workloads.generic_matrix(B, I, seed=410 + B)
    say(f"int4 matmul f32 chunks B={B}")
    Y = host(qt.qt_matmul_i4(dev(po), dev(so), O, I, dev(X)))
    yr, ar = _matmul_ref(po, so, O, I, X)
    assert componentwise_err(Y, yr, ar) <= TOL_F32


@pytest.mark.parametrize("B", [1, 7, 16, 33])
def test_i4_matmul_bf16(B):
    O, I = 50, 300
    so, po = _i4_packed_for(O, I, seed=200 + B)
    Xb = workloads.bf16_bits_rne(workloads.generic_matrix(B, I, seed=B + 9))
    say(f"int4 matmul bf16 B={B}")
    Y = host(qt.qt_matmul_i4(dev(po), dev(so), O, I, dev_bf16(Xb)))
    yr, ar = _matmul_ref(po, so, O, I, workloads.bf16_bits_to_f32(Xb))
    assert componentwise_err(Y, yr, ar) <= TOL_F32


def test_i4_matmul_b1_equals_matvec():
    O, I = 100, 777
    so, po = _i4_packed_for(O, I, seed=5)
    x = workloads.generic_vector(I, seed=6)
    y1 = host(qt.qt_matvec_i4(dev(po), dev(so), O, I, dev(x)))
    y2 = host(qt.qt_matmul_i4(dev(po), dev(so), O, I, dev(x[None, :])))
    assert np.array_equal(bits(y1), bits(y2[0]))


def test_i4_reconstruction_beats_int3_on_the_same_weights():
    # one more bit per weight: the GPU's int4 reconstruction error is below
    # its int3-g64 error on every row of the decode matrix's first 64 rows
    W, _ = workloads.decode(False)
    W = np.ascontiguousarray(W[:64])
    O, I = W.shape
    s4, c4, _ = qt.qt_quantize_g64_i4(dev(W))
    s3, c3, _ = qt.qt_quantize_g64(dev(W))
    r4 = np.repeat(host(s4).astype(np.float64), 64, axis=1)[:, :I] * host(c4) - W
    r3 = np.repeat(host(s3).astype(np.float64), 64, axis=1)[:, :I] * host(c3) - W
    assert np.all((r4 ** 2).sum(axis=1) < (r3 ** 2).sum(axis=1))


# ---------------------------------------------------------------- grouped (MoE)
def _grouped_i4_case(E, O, I, T, topk, seed):
    rng = workloads.rng_for("generic", 900 + seed, E, O, I)
    logits = rng.random((T, E))
    top = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    tok, exp, offs = workloads.route_pairs(top, E)
    Ws = [workloads.generic_weights(O, I, seed=3000 * seed + e) for e in range(E)]
    q = [oracle.quantize_g64_i4(w) for w in Ws]
    so = np.stack([a[0] for a in q])
    po = np.stack([oracle.pack_i4(a[1]) for a in q])
    X = workloads.generic_matrix(T, I, seed=seed + 50)
    return tok, exp, offs, so, po, X


@pytest.mark.parametrize("E,O,I,T,topk", [(4, 40, 300, 6, 2), (16, 64, 1000, 32, 8),
                                          (3, 100, 64, 40, 3), (8, 33, 7200, 5, 1),
                                          (5, 130, 450, 12, 3), (3, 70, 130, 9, 2),
                                          (2, 65, 97, 7, 2)])
def test_i4_grouped_matvec(E, O, I, T, topk):
    tok, exp, offs, so, po, X = _grouped_i4_case(E, O, I, T, topk, seed=E + T)
    P = tok.size
    say(f"int4 grouped E={E} O={O} I={I} P={P}")
    Y = host(qt.qt_matvec_i4_grouped(dev(po), dev(so), E, O, I, dev(X), dev(offs), P,
                                     pair_row=dev(tok)))
    for p in range(P):
        e, t = exp[p], tok[p]
        yr, ar = matvec_ref(po[e], so[e], O, I, X[t])
        assert componentwise_err(Y[p], yr, ar) <= TOL_F32, (p, e, t)
    H = workloads.generic_matrix(P, I, seed=78)
    Y2 = host(qt.qt_matvec_i4_grouped(dev(po), dev(so), E, O, I, dev(H), dev(offs), P))
    for p in range(P):
        yr, ar = matvec_ref(po[exp[p]], so[exp[p]], O, I, H[p])
        assert componentwise_err(Y2[p], yr, ar) <= TOL_F32


def test_i4_grouped_one_hot_is_exact_and_empty_experts():
    # one-hot inputs pick single codes: v * s exactly, through the v/16 entry
    # and the final scaling by 16
    E, O, I = 4, 70, 200
    offs = np.array([0, 0, 5, 5, 5], np.int32)
    Ws = [workloads.generic_weights(O, I, seed=40 + e) for e in range(E)]
    q = [oracle.quantize_g64_i4(w) for w in Ws]
    so = np.stack([a[0] for a in q])
    po = np.stack([oracle.pack_i4(a[1]) for a in q])
    cols = [0, 1, 63, 64, 199]
    X = np.zeros((5, I), np.float32)
    for p, i in enumerate(cols):
        X[p, i] = 1.0
    say("int4 grouped one-hot")
    Y = host(qt.qt_matvec_i4_grouped(dev(po), dev(so), E, O, I, dev(X), dev(offs), 5))
    c1, s1 = q[1][1], q[1][0]
    for p, i in enumerate(cols):
        assert np.array_equal(Y[p], s1[:, i // 64] * c1[:, i].astype(np.float32))


def test_mixed_bits_moe_step_up_int3_down_int4():
    # the per-projection mix: up at int3-g64, down at grouped int4, on one
    # routing; each projection against the oracle of its own format
    E, T, topk, D, F = 8, 12, 2, 640, 256
    rng = workloads.rng_for("generic", 4242)
    top = np.argsort(-rng.random((T, E)), axis=1, kind="stable")[:, :topk].astype(np.int32)
    tok, exp, offs = workloads.route_pairs(top, E)
    P = tok.size
    up = [oracle.quantize_g64(workloads.generic_weights(F, D, seed=60 + e)) for e in range(E)]
    dn = [oracle.quantize_g64_i4(workloads.generic_weights(D, F, seed=80 + e))
          for e in range(E)]
    su = np.stack([a[0] for a in up])
    pu = np.stack([oracle.pack_i3(a[1]) for a in up])
    sdn = np.stack([a[0] for a in dn])
    pdn = np.stack([oracle.pack_i4(a[1]) for a in dn])
    X = workloads.generic_matrix(T, D, seed=91)
    H = workloads.generic_matrix(P, F, seed=92)  # the down projection's own inputs
    say(f"mixed-bit MoE step E={E} P={P}")
    Yu = host(qt.qt_matvec_i3_grouped(dev(pu), dev(su), E, F, D, dev(X), dev(offs), P,
                                      pair_row=dev(tok)))
    Yd = host(qt.qt_matvec_i4_grouped(dev(pdn), dev(sdn), E, D, F, dev(H), dev(offs), P))
    for p in range(P):
        e = exp[p]
        yr, ar = oracle.matvec_f64(pu[e], su[e], F, D, X[tok[p]])
        assert componentwise_err(Yu[p], yr, ar) <= TOL_F32
        yr, ar = matvec_ref(pdn[e], sdn[e], D, F, H[p])
        assert componentwise_err(Yd[p], yr, ar) <= TOL_F32
