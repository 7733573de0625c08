"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: each check is a hand-derived
byte pattern, a closed form, a library routine (numpy), a brute-force search in
another precision, or an invariant of the method.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from tests.parity import componentwise_err, np_decode_planes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_facts():
    facts = {}
    for line in open(os.path.join(GOLDEN, "format_facts.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            facts[k] = float(v)
    return facts


def _codes_from_rule(rule, n):
    if rule == "mod8":
        return np.array([(j % 8) - 4 for j in range(n)], np.int8)
    if rule.startswith("list:"):
        vals = [int(t) for t in rule[5:].split(",")]
        return np.array(vals + [0] * (n - len(vals)), np.int8)
    parts = rule.split(",")
    base = int(parts[0].split(":")[1])
    c = np.full(n, base, np.int8)
    for p in parts[1:]:
        j, v = p.split(":")
        c[int(j)] = int(v)
    return c


def _read_pack_examples():
    out = []
    for line in open(os.path.join(GOLDEN, "pack_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, n, rule, hexbytes = [t.strip() for t in line.split("|")]
        out.append((name, int(n), rule, bytes.fromhex(hexbytes.replace(" ", ""))))
    return out


# ---------------------------------------------------------------- format facts
def test_format_sizes_match_pages():
    f = _read_facts()
    for O, I in [(1, 64), (3, 65), (256, 512), (2048, 7168), (2048, 7200), (7, 1)]:
        G = -(-I // 64)
        assert oracle.groups(I) == G
        assert oracle.packed_bytes(O, I) == O * G * int(f["bytes_per_group"])
    assert f["low_plane_bytes"] + f["high_plane_bytes"] == f["bytes_per_group"]
    # 24 B of codes + a 4 B f32 scale per 64 weights = 3.5 bits per weight
    assert (f["bytes_per_group"] + 4) * 8 / f["group_size"] == f["bits_per_weight_with_scale"]


@pytest.mark.parametrize("ex", _read_pack_examples(), ids=lambda e: e[0])
def test_pack_worked_examples(ex):
    name, n, rule, expect = ex
    codes = _codes_from_rule(rule, n)[None, :]
    packed = oracle.pack_i3(codes)
    assert packed.tobytes() == expect, (name, packed.tobytes().hex())
    assert np.array_equal(oracle.unpack_i3(packed, 1, n), codes)


def test_pack_every_position_and_code():
    # 64 positions x 8 codes: one slot differs from a background, every bit
    # position of both planes is exercised, and the decoded group must match
    # the numpy-unpackbits decoder as well as the oracle's own unpacker.
    for bg in (-4, 0, 3):
        rows = []
        for j in range(64):
            for v in range(-4, 4):
                c = np.full(64, bg, np.int8)
                c[j] = v
                rows.append(c)
        codes = np.stack(rows)
        packed = oracle.pack_i3(codes)
        assert np.array_equal(oracle.unpack_i3(packed, codes.shape[0], 64), codes)
        assert np.array_equal(np_decode_planes(packed, codes.shape[0], 64), codes)


@pytest.mark.parametrize("I", [1, 7, 63, 64, 65, 100, 128, 200, 7200])
def test_pack_roundtrip_random_and_tail_padding(I):
    rng = workloads.rng_for("generic", 77, I)
    O = 5
    codes = rng.integers(-4, 4, size=(O, I)).astype(np.int8)
    packed = oracle.pack_i3(codes)
    assert packed.size == O * (-(-I // 64)) * 24
    assert np.array_equal(oracle.unpack_i3(packed, O, I), codes)
    assert np.array_equal(np_decode_planes(packed, O, I), codes)
    # padding slots of a tail group decode as v = 0 (u = 4)
    G = -(-I // 64)
    full = np_decode_planes(packed, O, G * 64)
    assert np.all(full[:, I:] == 0)


# ---------------------------------------------------------------- quantizer
def test_rtn_rounding_worked_example():
    # exact binary fractions: every quotient w/s is exact, so only the rounding
    # rule decides: 4 -> clamp 3, 2.5 -> 2 (ties to even), -3.5 -> -4, 1.5 -> 2
    w = np.zeros((1, 64), np.float32)
    w[0, :5] = [1.0, 0.625, -0.875, 0.375, -1.0]
    s, c, k = oracle.quantize_g64(w)
    assert s[0, 0] == np.float32(0.25)
    assert list(c[0, :5]) == [3, 2, -4, 2, -4]
    assert np.all(c[0, 5:] == 0) and k[0, 0] == 0


def test_rtn_matches_numpy_rint():
    # plain absmax/4 RTN reduces to IEEE f32 division and numpy.rint
    # (round half to even) followed by a clamp to [-4, 3]
    for I in (512, 100, 7200):
        W = workloads.generic_weights(33, I, seed=3)
        s, c, _ = oracle.quantize_g64(W)
        G = -(-I // 64)
        Wp = np.zeros((33, G * 64), np.float32)
        Wp[:, :I] = W
        amax = np.abs(Wp.reshape(33, G, 64)).max(axis=2).astype(np.float32)
        base = (amax * np.float32(0.25)).astype(np.float32)
        assert np.array_equal(s, base)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.rint(Wp.reshape(33, G, 64) / base[:, :, None])
        q = np.where(base[:, :, None] == 0, 0, np.clip(q, -4, 3)).reshape(33, G * 64)[:, :I]
        assert np.array_equal(c, q.astype(np.int8))


def test_codes_in_range_and_zero_groups():
    W = workloads.generic_weights(16, 300, seed=4)
    W[3] = 0.0
    W[5, 64:128] = 0.0
    d = np.abs(workloads.generic_vector(300, seed=5)) + 0.1
    s, c, k = oracle.quantize_g64(W, d=d, n_grid=64)
    assert c.min() >= -4 and c.max() <= 3
    assert np.all(s[3] == 0) and np.all(c[3] == 0) and np.all(k[3] == 0)
    assert s[5, 1] == 0 and np.all(c[5, 64:128] == 0) and k[5, 1] == 0


def _bruteforce_f64(w, d, n_grid, lo, hi):
    """Every candidate's objective in double precision: scales and codes as the
    method defines them, the weighted squared error summed in f64."""
    amax = np.float32(np.max(np.abs(w)))
    base = np.float32(amax * np.float32(0.25))
    fk = np.linspace(lo, hi, n_grid).astype(np.float32)
    E = np.empty(n_grid)
    for k in range(n_grid):
        s = np.float32(base * fk[k])
        q = np.clip(np.rint(w.astype(np.float64) / float(s)), -4, 3) if s != 0 else np.zeros_like(w, np.float64)
        r = w.astype(np.float64) - float(s) * q
        E[k] = np.sum(d.astype(np.float64) * r * r)
    return E


def test_search_against_f64_bruteforce():
    rng = workloads.rng_for("generic", 91)
    O, I = 40, 64 * 6
    W = workloads.generic_weights(O, I, seed=9)
    d = np.exp(rng.normal(size=I)).astype(np.float32)
    s, c, k, errs = oracle.quantize_g64(W, d=d, n_grid=64, return_errs=True)
    clear = 0
    for o in range(O):
        for g in range(I // 64):
            w = W[o, 64 * g:64 * g + 64]
            E = _bruteforce_f64(w, d[64 * g:64 * g + 64], 64, 0.5, 1.0)
            kk = int(k[o, g])
            # the chosen candidate is optimal up to f32 rounding of the objective
            assert E[kk] <= E.min() * (1 + 1e-5) + 1e-30
            srt = np.sort(E)
            if srt[1] > srt[0] * (1 + 1e-4):
                clear += 1
                assert kk == int(np.argmin(E))
            # the f32 objective agrees with the f64 one
            assert abs(float(errs[o, g, kk]) - E[kk]) <= 1e-5 * E[kk] + 1e-30
    assert clear > O  # most groups have an unambiguous optimum


def test_search_invariants():
    W = workloads.generic_weights(64, 512, seed=11)
    d = (np.abs(workloads.generic_vector(512, seed=12)) + 0.05).astype(np.float32)
    s, c, k, errs = oracle.quantize_g64(W, d=d, n_grid=64, return_errs=True)
    # never worse than plain RTN: k = 63 is the absmax/4 scale itself
    best = np.take_along_axis(errs, k[..., None].astype(np.int64), axis=2)[..., 0]
    assert np.all(best <= errs[..., 63])
    assert np.all(errs.min(axis=2) == best)
    # the k=63 candidate is bit-identical to the no-search scale
    assert oracle.grid_factor(63, 64, 0.5, 1.0) == 1.0
    s0, c0, _ = oracle.quantize_g64(W)
    s63, c63, _ = oracle.quantize_g64(W, d=d, n_grid=64)
    m = k == 63
    assert np.array_equal(s63[m], s0[m])
    # unit weights are the unweighted search
    s1, c1, k1 = oracle.quantize_g64(W, d=np.ones(512, np.float32), n_grid=64)
    s2, c2, k2 = oracle.quantize_g64(W, d=None, n_grid=64)
    assert np.array_equal(k1, k2) and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # scaling d by a power of two is exact and cannot change the choice
    s3, c3, k3 = oracle.quantize_g64(W, d=d * np.float32(8.0), n_grid=64)
    assert np.array_equal(k3, k) and np.array_equal(c3, c)
    # scaling W by a power of two scales the scales and keeps codes and choices
    s4, c4, k4 = oracle.quantize_g64(W * np.float32(4.0), d=d, n_grid=64)
    assert np.array_equal(k4, k) and np.array_equal(c4, c) and np.array_equal(s4, s * np.float32(4.0))
    # ties go to the lowest k: a group of equal magnitudes +-a has E = 0 for
    # every scale that maps a onto a code exactly; all-equal |w| = a gives
    # q = -4 exactly only for s = a/4 (k = 63)
    w = np.full((1, 64), 0.5, np.float32)
    w[0, ::2] = -0.5
    sw, cw, kw, ew = oracle.quantize_g64(w, n_grid=64, return_errs=True)
    assert kw[0, 0] == int(np.argmin(ew[0, 0]))


def test_search_worked_example_s():
    # a fixed deterministic group: evenly spread magnitudes plus one large
    # value; the f64 brute force must pick the same candidate, with and
    # without non-uniform importance
    j = np.arange(64)
    w = (((37 * j) % 64 - 31.5) / 64 * 0.05).astype(np.float32)
    w[9] = np.float32(0.09)
    for d in (np.ones(64, np.float32), (4.0 ** (j % 3)).astype(np.float32)):
        s, c, k = oracle.quantize_g64(w[None, :], d=d, n_grid=64)
        E = _bruteforce_f64(w, d, 64, 0.5, 1.0)
        assert int(k[0, 0]) == int(np.argmin(E))
        assert s[0, 0] == np.float32(np.float32(np.max(np.abs(w)) * np.float32(0.25))
                                     * np.linspace(0.5, 1.0, 64).astype(np.float32)[k[0, 0]])


def read_search_order_fixture():
    """The group of tests/golden/search_order.txt -> (w[64], d[64], n, lo, hi,
    expected k, expected scale, expected codes[64])."""
    w = np.zeros(64, np.float32)
    d = np.ones(64, np.float32)
    codes = np.zeros(64, np.int8)
    for line in open(os.path.join(GOLDEN, "search_order.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = [t.strip() for t in line.split("|")]
        if f[0] == "grid":
            n, lo, hi = int(f[1]), float(f[2]), float(f[3])
        elif f[0] == "slot":
            w[int(f[1])] = np.float32(float(f[2]))
            d[int(f[1])] = np.float32(float(f[3]))
        elif f[0] == "expect":
            k, scale = int(f[1]), np.float32(float(f[2]))
            for item in f[3].split(","):
                j, v = item.split(":")
                codes[int(j)] = int(v)
    return w, d, n, lo, hi, k, scale, codes


def test_search_summation_order_worked_example():
    # pins the halving order of the objective's sum (a left-to-right sum picks
    # the other candidate on this group; derivation in the fixture)
    w, d, n, lo, hi, k, scale, codes = read_search_order_fixture()
    s, c, kk, errs = oracle.quantize_g64(w[None, :], d=d, n_grid=n, lo=lo, hi=hi,
                                         return_errs=True)
    assert errs[0, 0, 0] == np.float32(1.0 + 2.0 ** -23)
    assert errs[0, 0, 1] == np.float32(1.0)
    assert int(kk[0, 0]) == k and s[0, 0] == scale
    assert np.array_equal(c[0], codes)


# ---------------------------------------------------------------- signed two-stage search
def _err_f64(w, d, s):
    """The objective for one scale in f64 (codes as the method decides them:
    the f32 quotient rounded to nearest even, clamped)."""
    s = np.float32(s)
    if s == 0:
        q = np.zeros_like(w, np.float64)
    else:
        q = np.clip(np.rint((w / s).astype(np.float32)).astype(np.float64), -4, 3)
    r = w.astype(np.float64) - float(s) * q
    return float(np.sum(d.astype(np.float64) * r * r))


def test_signed_search_worked_example():
    # w = (4, 0, ..., 0): base = 1.  Positive scales put 4 on code 3 at best
    # (f = 1: error (4 - 3)^2 = 1); the scale -1 puts it on -4 exactly
    # (error 0), which a signed search must find; the refinement keeps it.
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = 4.0
    for n2 in (0, 32):
        s, c = oracle.quantize_g64_signed(w, None, 64, n2)
        assert s[0, 0] == np.float32(-1.0) and c[0, 0] == -4 and np.all(c[0, 1:] == 0)
    su, cu, _ = oracle.quantize_g64(w, None, 64)
    assert su[0, 0] == np.float32(1.0) and cu[0, 0] == 3
    # an all-zero group: scale +0, codes 0
    z = np.zeros((1, 70), np.float32)
    s, c = oracle.quantize_g64_signed(z, None, 64, 32)
    assert np.all(s == 0) and not np.any(np.signbit(s)) and np.all(c == 0)


def test_signed_stage1_against_f64_bruteforce():
    # stage 1 alone (n2 = 0) is the best of 2 x 64 signed candidates
    rng = workloads.rng_for("generic", 92)
    O, I = 30, 64 * 4
    W = workloads.generic_weights(O, I, seed=21)
    d = np.exp(rng.normal(size=I)).astype(np.float32)
    s, c = oracle.quantize_g64_signed(W, d, 64, 0)
    fk = np.linspace(0.5, 1.0, 64).astype(np.float32)
    clear = 0
    for o in range(O):
        for g in range(I // 64):
            w, dg = W[o, 64 * g:64 * g + 64], d[64 * g:64 * g + 64]
            base = np.float32(np.float32(np.max(np.abs(w))) * np.float32(0.25))
            cands = [np.float32(sg * np.float32(base * f)) for f in fk for sg in (1, -1)]
            E = np.array([_err_f64(w, dg, x) for x in cands])
            e = _err_f64(w, dg, s[o, g])
            assert e <= E.min() * (1 + 1e-5) + 1e-30
            srt = np.sort(E)
            if srt[1] > srt[0] * (1 + 1e-4):
                clear += 1
                assert s[o, g] == cands[int(np.argmin(E))]
    assert clear > O


def test_signed_search_invariants():
    W = workloads.generic_weights(48, 64 * 5 + 20, seed=23)
    I = W.shape[1]
    d = (np.abs(workloads.generic_vector(I, seed=24)) + 0.05).astype(np.float32)
    s1, c1 = oracle.quantize_g64_signed(W, d, 64, 0)
    s2, c2 = oracle.quantize_g64_signed(W, d, 64, 32)
    su, cu, _ = oracle.quantize_g64(W, d=d, n_grid=64)
    G = s2.shape[1]
    fk = np.linspace(0.5, 1.0, 64).astype(np.float32)
    for o in range(W.shape[0]):
        for g in range(G):
            lo_, hi_ = 64 * g, min(64 * g + 64, I)
            w, dg = W[o, lo_:hi_], d[lo_:hi_]
            e_u = _err_f64(w, dg, su[o, g])
            e_1 = _err_f64(w, dg, s1[o, g])
            e_2 = _err_f64(w, dg, s2[o, g])
            # each stage can only improve (up to f32 rounding of the objective)
            assert e_1 <= e_u * (1 + 1e-5) + 1e-30
            assert e_2 <= e_1 * (1 + 1e-5) + 1e-30
            # a refined scale keeps the stage-1 sign and lies between the
            # stage-1 winner's neighbours on the grid
            assert np.signbit(s2[o, g]) == np.signbit(s1[o, g])
            base = np.float32(np.float32(np.max(np.abs(w))) * np.float32(0.25))
            k = int(np.argmin(np.abs(np.abs(s1[o, g]) - base * fk)))
            a, b = fk[max(k - 1, 0)], fk[min(k + 1, 63)]
            assert base * a * (1 - 1e-6) <= abs(s2[o, g]) <= base * b * (1 + 1e-6)
            # codes are the rounding rule applied to the chosen scale
            q = np.clip(np.rint((w / s2[o, g]).astype(np.float32)), -4, 3)
            assert np.array_equal(c2[o, lo_:hi_], q.astype(np.int8))
    # negating W negates every scale and keeps the codes (the candidate set
    # holds both signs) wherever stage 1 has a unique winner
    s3, c3 = oracle.quantize_g64_signed(-W, d, 64, 0)
    same = s3 == -s1
    assert same.mean() > 0.95
    for o, g in zip(*np.nonzero(same)):
        assert np.array_equal(c3[o, 64 * g:64 * g + 64], c1[o, 64 * g:64 * g + 64])


# ---------------------------------------------------------------- matvec / matmul
def _quantized(O, I, seed):
    W = workloads.generic_weights(O, I, seed=seed)
    s, c, _ = oracle.quantize_g64(W)
    return s, c, oracle.pack_i3(c)


@pytest.mark.parametrize("O,I", [(8, 64), (17, 100), (64, 7168), (5, 7200), (3, 1)])
def test_matvec_f64_against_numpy(O, I):
    s, c, p = _quantized(O, I, seed=O + I)
    x = workloads.generic_vector(I, seed=I)
    y, a = oracle.matvec_f64(p, s, O, I, x)
    G = -(-I // 64)
    v = np_decode_planes(p, O, I).astype(np.float64)
    what = v * np.repeat(s.astype(np.float64), 64, axis=1)[:, :I]
    assert np.allclose(oracle.dequant_f64(p, s, O, I), what, rtol=0, atol=0)
    yr = what @ x.astype(np.float64)
    ar = np.abs(what * x.astype(np.float64)[None, :]).sum(axis=1)
    assert componentwise_err(y, yr, ar) < 1e-13
    assert np.allclose(a, ar, rtol=1e-13, atol=0)
    # the f32 per-group path is within f32 rounding of the f64 reference
    yf = oracle.matvec_f32(p, s, O, I, x)
    assert componentwise_err(yf, yr, ar) < 1e-5


def test_matvec_one_hot_closed_form():
    O, I = 9, 200
    s, c, p = _quantized(O, I, seed=5)
    for i in (0, 63, 64, 150, 199):
        x = np.zeros(I, np.float32)
        x[i] = 1.0
        y, _ = oracle.matvec_f64(p, s, O, I, x)
        exp = s[:, i // 64].astype(np.float64) * c[:, i].astype(np.float64)
        assert np.array_equal(y, exp)
        assert np.array_equal(oracle.matvec_f32(p, s, O, I, x), (s[:, i // 64] * c[:, i].astype(np.float32)))


def test_matvec_zero_weights():
    O, I = 4, 130
    s, c, _ = oracle.quantize_g64(np.zeros((O, I), np.float32))
    p = oracle.pack_i3(c)
    y, a = oracle.matvec_f64(p, s, O, I, workloads.generic_vector(I))
    assert np.all(y == 0) and np.all(a == 0)


def test_matmul_sampled_matches_matvec_rows():
    O, I, B = 12, 300, 5
    s, c, p = _quantized(O, I, seed=6)
    X = workloads.generic_matrix(B, I, seed=6)
    t_idx = np.repeat(np.arange(B), O)
    o_idx = np.tile(np.arange(O), B)
    y, a = oracle.matmul_f64_sampled(p, s, O, I, X, t_idx, o_idx)
    what = oracle.dequant_f64(p, s, O, I)
    Yr = X.astype(np.float64) @ what.T
    Ar = (np.abs(X.astype(np.float64))[:, None, :] * np.abs(what)[None, :, :]).sum(axis=2)
    assert np.allclose(a, Ar.reshape(-1), rtol=1e-13, atol=0)
    assert componentwise_err(y, Yr.reshape(-1), Ar.reshape(-1)) < 1e-13
    assert np.allclose(y, Yr.reshape(-1), rtol=1e-12, atol=1e-15)
    for t in range(B):
        yt, _ = oracle.matvec_f64(p, s, O, I, X[t])
        assert np.array_equal(yt, y[t * O:(t + 1) * O])


# ---------------------------------------------------------------- Hessian diagonal
def test_hessian_diag_closed_form_and_numpy():
    T, I = 37, 50
    cst = workloads.generic_vector(I, seed=8)
    X = np.tile(cst, (T, 1))
    d = oracle.hessian_diag(X)
    assert np.allclose(d, T * cst.astype(np.float64) ** 2, rtol=1e-15, atol=0)
    assert np.array_equal(oracle.hessian_diag(np.ones((T, I), np.float32)), np.full(I, float(T)))
    X = workloads.generic_matrix(T, I, seed=9)
    ref = np.einsum("ti,ti->i", X.astype(np.float64), X.astype(np.float64))
    assert np.allclose(oracle.hessian_diag(X), ref, rtol=1e-14, atol=0)
    # accumulation over two halves equals one pass
    d1 = oracle.hessian_diag(X[:20])
    d2 = oracle.hessian_diag(X[20:], d_in=d1)
    assert np.allclose(d2, ref, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- outlier invariant
def _rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def test_outlier_rows_int3_g64_beats_rowwise_int4_tiny():
    # pull request page, "Tests": on outlier rows the int3-g64 reconstruction
    # RMS is below per-row int4 (pooled over the 4 outlier rows of the Tiny set)
    W, x, rows = workloads.tiny()
    s, c, _ = oracle.quantize_g64(W)
    p = oracle.pack_i3(c)
    O, I = W.shape
    r3 = oracle.dequant_f64(p, s, O, I)[rows] - W[rows].astype(np.float64)
    r4 = oracle.rowint_recon(W, 4)[rows] - W[rows].astype(np.float64)
    assert _rms(r3) < _rms(r4), (_rms(r3), _rms(r4))


def test_outlier_rows_int3_g64_beats_rowwise_int4_wide():
    # the same property at the I = 7168 width of the page's own test shape,
    # where it is robust (8 outliers x20 per row)
    rng = workloads.rng_for("generic", 4242)
    O, I = 16, 7168
    W = rng.normal(0, 0.02, size=(O, I))
    for r in range(O):
        cols = rng.choice(I, 8, replace=False)
        W[r, cols] *= 20
    W = W.astype(np.float32)
    s, c, _ = oracle.quantize_g64(W)
    p = oracle.pack_i3(c)
    r3 = oracle.dequant_f64(p, s, O, I) - W.astype(np.float64)
    r4 = oracle.rowint_recon(W, 4) - W.astype(np.float64)
    ratio = _rms(r4) / _rms(r3)
    assert ratio > 2.0, ratio
    for o in range(O):
        assert _rms(r3[o]) < _rms(r4[o])


def test_rowint_matches_numpy():
    W = workloads.generic_weights(7, 90, seed=10)
    amax = np.abs(W).max(axis=1).astype(np.float32)
    s = (amax / np.float32(8)).astype(np.float32)
    q = np.clip(np.rint(W / s[:, None]), -8, 7)
    assert np.array_equal(oracle.rowint_recon(W, 4), s[:, None].astype(np.float64) * q)


# ---------------------------------------------------------------- grouped int4
def _np_decode_nibbles(packed, O, I):
    """Independent decoder of the grouped int4 layout: 32 bytes per group,
    code j in the low nibble of byte j/2 (even j) or the high nibble (odd j),
    stored as v + 8."""
    G = -(-I // 64)
    b = np.asarray(packed, np.uint8).reshape(O, G, 32)
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(O, G * 64)
    return nib[:, :I].astype(np.int16) - 8


def test_i4_format_and_worked_bytes():
    assert oracle.packed_bytes_i4(3, 64) == 96 and oracle.packed_bytes_i4(2, 70) == 128
    # v_j = (j mod 16) - 8: u_j = j mod 16, byte b = u_{2b} | u_{2b+1} << 4
    c = ((np.arange(64) % 16) - 8).astype(np.int8)[None, :]
    p = oracle.pack_i4(c)
    assert list(p[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(p[8:16], p[:8]) and np.array_equal(p[:16], p[16:32])
    # a short tail group: 6 real codes (v = 7), the rest padded with v = 0
    t = np.zeros((1, 70), np.int8)
    t[0, 64:] = 7
    q = oracle.pack_i4(t)
    assert list(q[32:35]) == [0xFF, 0xFF, 0xFF] and np.all(q[35:64] == 0x88)
    assert np.all(q[:32] == 0x88)


def test_i4_every_position_and_code_roundtrip():
    for v in range(-8, 8):
        for j in range(64):
            c = np.zeros((1, 64), np.int8)
            c[0, j] = v
            p = oracle.pack_i4(c)
            assert np.array_equal(oracle.unpack_i4(p, 1, 64), c)
            assert np.array_equal(_np_decode_nibbles(p, 1, 64), c.astype(np.int16))


def test_i4_rtn_rounding_and_clamps():
    # base = absmax/8 = 1 for absmax 8: quotients equal the weights
    w = np.array([[8.0, 7.5, 6.5, -7.5, -8.0, 0.5, -0.5, 2.5] + [0.0] * 56], np.float32)
    s, c, k = oracle.quantize_g64_i4(w)
    assert s[0, 0] == np.float32(1.0)
    # 8 -> 7 (clip), 7.5 -> 8 -> 7, 6.5 -> 6 (ties to even), -7.5 -> -8,
    # -8 -> -8, 0.5 -> 0, -0.5 -> -0, 2.5 -> 2
    assert list(c[0, :8]) == [7, 7, 6, -8, -8, 0, 0, 2]
    W = workloads.generic_weights(20, 200, seed=31)
    s, c, _ = oracle.quantize_g64_i4(W)
    G = -(-200 // 64)
    for g in range(G):
        blk = W[:, 64 * g:64 * g + 64]
        base = (np.max(np.abs(blk), axis=1) * np.float32(0.125)).astype(np.float32)
        assert np.array_equal(s[:, g], base)
        q = np.clip(np.rint((blk / base[:, None]).astype(np.float32)), -8, 7)
        assert np.array_equal(c[:, 64 * g:64 * g + blk.shape[1]], q.astype(np.int8))


def test_i4_search_against_f64_bruteforce():
    rng = workloads.rng_for("generic", 93)
    O, I = 24, 64 * 3
    W = workloads.generic_weights(O, I, seed=33)
    d = np.exp(rng.normal(size=I)).astype(np.float32)
    s, c, k = oracle.quantize_g64_i4(W, d, 64, 0.5, 1.0)
    fk = np.linspace(0.5, 1.0, 64).astype(np.float32)
    clear = 0
    for o in range(O):
        for g in range(I // 64):
            w, dg = W[o, 64 * g:64 * g + 64], d[64 * g:64 * g + 64]
            base = np.float32(np.float32(np.max(np.abs(w))) * np.float32(0.125))
            E = []
            for f in fk:
                sc = np.float32(base * f)
                q = np.clip(np.rint((w / sc).astype(np.float32)).astype(np.float64), -8, 7)
                r = w.astype(np.float64) - float(sc) * q
                E.append(float(np.sum(dg.astype(np.float64) * r * r)))
            E = np.array(E)
            kk = int(k[o, g])
            assert E[kk] <= E.min() * (1 + 1e-5) + 1e-30
            srt = np.sort(E)
            if srt[1] > srt[0] * (1 + 1e-4):
                clear += 1
                assert kk == int(np.argmin(E))
    assert clear > O


def test_i4_reconstruction_beats_int3_and_rowwise_int4():
    # one more bit per weight: lower error than int3-g64 on the same groups;
    # group scales: lower error than per-row int4 on the outlier rows
    W, _, rows = workloads.tiny()
    O, I = W.shape
    s4, c4, _ = oracle.quantize_g64_i4(W)
    r4 = c4.astype(np.float64) * np.repeat(s4.astype(np.float64), 64, axis=1)[:, :I] - W
    s3, c3, _ = oracle.quantize_g64(W)
    r3 = c3.astype(np.float64) * np.repeat(s3.astype(np.float64), 64, axis=1)[:, :I] - W
    rr = oracle.rowint_recon(W, 4) - W
    rms = lambda a: float(np.sqrt(np.mean(a ** 2)))
    assert rms(r4) < rms(r3)
    assert rms(r4[rows]) < rms(rr[rows])


@pytest.mark.parametrize("O,I", [(8, 64), (17, 100), (5, 7200)])
def test_i4_matvec_f64_against_numpy(O, I):
    W = workloads.generic_weights(O, I, seed=O * I)
    s, c, _ = oracle.quantize_g64_i4(W)
    p = oracle.pack_i4(c)
    x = workloads.generic_vector(I, seed=I + 1)
    y, a = oracle.matvec_i4_f64(p, s, O, I, x)
    what = _np_decode_nibbles(p, O, I).astype(np.float64) * np.repeat(
        s.astype(np.float64), 64, axis=1)[:, :I]
    yr = what @ x.astype(np.float64)
    ar = np.abs(what * x.astype(np.float64)[None, :]).sum(axis=1)
    assert componentwise_err(y, yr, ar) < 1e-13
    assert np.allclose(a, ar, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- GPTQ / LDLQ
def _correlated_x(T, I, seed):
    # tokens with correlated features: Z M, M a random mixing matrix plus the
    # identity, and lognormal column scales (the search workload's recipe)
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((T, I))
    M = np.eye(I) + 0.3 * rng.standard_normal((I, I)) / np.sqrt(I)
    c = np.exp(rng.standard_normal(I))
    return ((Z @ M) * c).astype(np.float32)


def test_hessian_full_against_numpy_and_the_diagonal():
    X = _correlated_x(300, 72, 1)
    H = oracle.hessian_full(X)
    X64 = X.astype(np.float64)
    assert np.allclose(H, X64.T @ X64, rtol=1e-12, atol=1e-9)
    assert np.array_equal(H, H.T)
    d = oracle.hessian_diag(X)
    assert np.allclose(np.diag(H), d, rtol=1e-6)


def test_gptq_factor_two_by_two_closed_form():
    # A = [[5, 2], [2, 4]] (no damping): A^-1 = [[4, -2], [-2, 5]] / 16, whose
    # upper Cholesky factor is U = [[1/2, -1/4], [0, 1/2]] (U^T U = A^-1)
    U = oracle.gptq_factor(np.array([[5.0, 2.0], [2.0, 4.0]]), 0.0)
    assert U.tolist() == [[0.5, -0.25], [0.0, 0.5]]


@pytest.mark.parametrize("damp", [0.0, 0.01])
def test_gptq_factor_against_numpy(damp):
    X = _correlated_x(400, 96, 2)
    H = X.astype(np.float64).T @ X.astype(np.float64)
    U = oracle.gptq_factor(H, damp)
    A = H + damp * np.mean(np.diag(H)) * np.eye(96)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    Un = np.linalg.cholesky(np.linalg.inv(A)).T
    assert np.abs(U - Un).max() <= 1e-9 * np.abs(Un).max()
    assert np.abs(U.T @ U @ A - np.eye(96)).max() <= 1e-9


def test_gptq_factor_rejects_an_indefinite_matrix():
    with pytest.raises(ValueError):
        oracle.gptq_factor(np.array([[1.0, 2.0], [2.0, 1.0]]), 0.0)


def test_gptq_with_a_diagonal_hessian_is_plain_rtn():
    # a diagonal H has a diagonal U: nothing propagates, every column is
    # rounded as it is
    W = workloads.generic_weights(20, 300, seed=8)
    H = np.diag(np.exp(np.random.default_rng(3).standard_normal(300)))
    U = oracle.gptq_factor(H, 0.01)
    assert not np.triu(U, 1).any()
    s, c = oracle.gptq_i3(W, U.astype(np.float32), 128)
    s0, c0, _ = oracle.quantize_g64(W)
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    assert np.array_equal(c, c0)


def test_gptq_two_column_worked_example():
    # A = [[5, 2], [2, 4]]: U = [[1/2, -1/4], [0, 1/2]].  W = [1, 5/16]: the
    # group scale is absmax/4 = 1/4; column 0 rounds 4 -> clamps to 3, scaled
    # error (1 - 3/4) / (1/2) = 1/2; column 1 becomes 5/16 - 1/2 * (-1/4) =
    # 7/16 = 1.75 s -> code 2 (plain RTN would give 1)
    U = oracle.gptq_factor(np.array([[5.0, 2.0], [2.0, 4.0]]), 0.0).astype(np.float32)
    W = np.array([[1.0, 0.3125]], np.float32)
    s, c = oracle.gptq_i3(W, U, 128)
    assert s[0, 0] == 0.25
    assert c.tolist() == [[3, 2]]
    assert oracle.quantize_g64(W)[1].tolist() == [[3, 1]]


def _classical_gptq(W, U):
    """The GPTQ sweep written out in numpy f64, unblocked (scales rounded to
    f32 as the rounder stores them): -> scales, codes, decision values."""
    Wc = W.astype(np.float64).copy()
    O, I = W.shape
    G = (I + 63) // 64
    codes = np.zeros((O, I), np.int8)
    scales = np.zeros((O, G), np.float32)
    vals = np.zeros((O, I))
    s = None
    for i in range(I):
        if i % 64 == 0:
            s = (np.abs(Wc[:, i:i + 64]).max(axis=1) * 0.25).astype(np.float32)
            scales[:, i // 64] = s
        sd = s.astype(np.float64)
        vals[:, i] = Wc[:, i]
        q = np.where(sd > 0, np.clip(np.rint(Wc[:, i] / np.where(sd > 0, sd, 1)), -4, 3), 0)
        codes[:, i] = q
        err = (Wc[:, i] - sd * q) / U[i, i]
        Wc[:, i + 1:] -= err[:, None] * U[i, i + 1:][None, :]
    return scales, codes, vals


def test_gptq_replay_agrees_with_a_numpy_sweep():
    X = _correlated_x(500, 160, 4)
    H = X.astype(np.float64).T @ X.astype(np.float64)
    U = oracle.gptq_factor(H, 0.01)
    W = workloads.generic_weights(24, 160, seed=9)
    sc, cc, vals = _classical_gptq(W, U)
    wt, base = oracle.gptq_replay(W, U.astype(np.float32), sc, cc)
    assert np.abs(wt - vals).max() <= 1e-5 * np.abs(W).max()
    assert np.allclose(base, sc, rtol=1e-5)


def _valid_against_replay(W, U32, s, c, tol=1e-4):
    """Every code rounds its column's replayed value and every scale is the
    replayed group base, up to f32-versus-f64 differences of the sweep."""
    wt, base = oracle.gptq_replay(W, U32, s, c)
    I = W.shape[1]
    sfull = np.repeat(s.astype(np.float64), 64, axis=1)[:, :I]
    assert np.allclose(s, base, rtol=1e-4, atol=1e-30), "scales are not the group bases"
    y = np.where(sfull > 0, wt / np.where(sfull > 0, sfull, 1), 0)
    cf = c.astype(np.float64)
    inner = (cf > -4) & (cf < 3)
    assert np.all(np.abs(y - cf)[inner] <= 0.5 + tol)
    assert np.all(y[cf == 3] >= 2.5 - tol) and np.all(y[cf == -4] <= -3.5 + tol)


@pytest.mark.parametrize("O,I", [(16, 64), (12, 200), (8, 333), (10, 512)])
def test_gptq_sweep_follows_the_algorithm(O, I):
    X = _correlated_x(600, I, 5 + I)
    H = X.astype(np.float64).T @ X.astype(np.float64)
    U32 = oracle.gptq_factor(H, 0.01).astype(np.float32)
    W = workloads.generic_weights(O, I, seed=I)
    s, c = oracle.gptq_i3(W, U32, 128)
    _valid_against_replay(W, U32, s, c)


def test_gptq_beats_rtn_on_correlated_inputs():
    for seed in (6, 7, 8):
        X = _correlated_x(800, 256, seed)
        H = X.astype(np.float64).T @ X.astype(np.float64)
        U = oracle.gptq_factor(H, 0.01)
        W = workloads.generic_weights(32, 256, seed=seed)
        s, c = oracle.gptq_i3(W, U.astype(np.float32), 128)
        s0, c0, _ = oracle.quantize_g64(W)
        H32 = H.astype(np.float32)
        n1, d1 = oracle.proxy_terms(W, c, s, H32)
        n0, d0 = oracle.proxy_terms(W, c0, s0, H32)
        assert d1 == d0
        assert n1 < n0, (seed, n1 / d1, n0 / d0)


def test_proxy_terms_against_numpy_and_the_weighted_objective():
    W = workloads.generic_weights(6, 130, seed=10)
    s, c, _ = oracle.quantize_g64(W)
    rng = np.random.default_rng(11)
    B = rng.standard_normal((130, 130)).astype(np.float32)
    H = (B @ B.T).astype(np.float32)
    num, den = oracle.proxy_terms(W, c, s, H)
    E = W.astype(np.float64) - np.repeat(s.astype(np.float64), 64, axis=1)[:, :130] * c
    H64 = H.astype(np.float64)
    assert np.isclose(num, np.einsum("oi,ij,oj->", E, H64, E), rtol=1e-12)
    assert np.isclose(den, np.einsum("oi,ij,oj->", W.astype(np.float64), H64, W), rtol=1e-12)
    # diagonal H: the numerator is the search objective summed over groups
    d = np.exp(rng.standard_normal(130)).astype(np.float32)
    num_d, _ = oracle.proxy_terms(W, c, s, np.diag(d))
    assert np.isclose(num_d, np.sum(E ** 2 * d[None, :]), rtol=1e-12)


# ---------------------------------------------------------------- MoE expert layer
def test_moe_route_worked_example():
    # logits [0.1, 0.5, 0.5, 0.2]: the two 0.5 tie (lower index first)
    e, w = oracle.moe_route(np.array([[0.1, 0.5, 0.5, 0.2]], np.float32), 2)
    assert e.tolist() == [[1, 2]] and np.allclose(w, [[0.5, 0.5]], rtol=0, atol=1e-15)
    e, w = oracle.moe_route(np.array([[0.1, 0.5, 0.5, 0.2]], np.float32), 3)
    assert e.tolist() == [[1, 2, 3]]
    # softmax of (0.5, 0.5, 0.2) in f64 of the f32 logits
    z = np.exp(np.float64(np.float32(0.2)) - np.float64(np.float32(0.5)))
    assert np.allclose(w, [[1 / (2 + z), 1 / (2 + z), z / (2 + z)]], rtol=1e-15)
    # equal logits, k = E: uniform weights, experts in index order
    e, w = oracle.moe_route(np.zeros((1, 5), np.float32), 5)
    assert e.tolist() == [[0, 1, 2, 3, 4]] and np.allclose(w, 0.2, rtol=1e-15)


def test_silu_closed_forms():
    assert oracle.silu_f64(0.0) == 0.0
    assert np.isclose(oracle.silu_f64(1.0), 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)
    assert oracle.silu_f64(-800.0) == -0.0 and oracle.silu_f64(800.0) == 800.0


def _moe_experts(E, F, D, seed, bits=(3, 3, 3)):
    out = []
    for which, (O, I), b in (("gate", (F, D), bits[0]), ("up", (F, D), bits[1]),
                             ("down", (D, F), bits[2])):
        ps, ss = [], []
        for e in range(E):
            W = workloads.generic_weights(O, I, seed=seed * 100 + e + (7 if which == "up" else 0)
                                          + (13 if which == "down" else 0))
            if b == 3:
                s, c, _ = oracle.quantize_g64(W)
                p = oracle.pack_i3(c)
            else:
                s, c, _ = oracle.quantize_g64_i4(W)
                p = oracle.pack_i4(c)
            ps.append(p)
            ss.append(s)
        out.append((np.stack(ps), np.stack(ss), b))
    return out


def test_moe_layer_properties():
    E, F, D, T, k = 6, 64, 128, 5, 2
    gate, up, down = _moe_experts(E, F, D, 1)
    X = workloads.generic_matrix(T, D, seed=2)
    logits = np.random.default_rng(3).random((T, E)).astype(np.float32)
    out, bound = oracle.moe_layer_f64(X, logits, k, gate, up, down)
    assert np.all(bound > 0)
    # zero gate weights: silu(0) = 0, so every output is exactly zero
    zg = (gate[0], np.zeros_like(gate[1]), 3)
    z, _ = oracle.moe_layer_f64(X, logits, k, zg, up, down)
    assert not z.any()
    # down scales doubled: the output doubles exactly
    d2 = (down[0], down[1] * 2, 3)
    o2, _ = oracle.moe_layer_f64(X, logits, k, gate, up, d2)
    assert np.array_equal(o2, 2 * out)
    # k = 1: the top expert alone, weight 1, against the dense formula
    o1, _ = oracle.moe_layer_f64(X, logits, 1, gate, up, down)
    e0 = np.argmax(logits, axis=1)
    for t in range(T):
        e = e0[t]
        Wg = oracle.dequant_f64(gate[0][e], gate[1][e], F, D)
        Wu = oracle.dequant_f64(up[0][e], up[1][e], F, D)
        Wd = oracle.dequant_f64(down[0][e], down[1][e], D, F)
        x = X[t].astype(np.float64)
        g = Wg @ x
        ref = Wd @ (g / (1 + np.exp(-g)) * (Wu @ x))
        assert np.allclose(o1[t], ref, rtol=1e-12, atol=1e-15)
    # relabelling the experts (and their logits) leaves the layer unchanged
    perm = np.random.default_rng(4).permutation(E)
    pg = (gate[0][perm], gate[1][perm], 3)
    pu = (up[0][perm], up[1][perm], 3)
    pd = (down[0][perm], down[1][perm], 3)
    op, _ = oracle.moe_layer_f64(X, logits[:, perm], k, pg, pu, pd)
    assert np.allclose(op, out, rtol=1e-12, atol=1e-15)


def test_dequant_f64_matches_matvec():
    W = workloads.generic_weights(9, 200, seed=5)
    s, c, _ = oracle.quantize_g64(W)
    p = oracle.pack_i3(c)
    x = workloads.generic_vector(200, seed=6)
    y, _ = oracle.matvec_f64(p, s, 9, 200, x)
    assert np.allclose(oracle.dequant_f64(p, s, 9, 200) @ x.astype(np.float64), y, rtol=1e-12)
    s4, c4, _ = oracle.quantize_g64_i4(W)
    p4 = oracle.pack_i4(c4)
    y4, _ = oracle.matvec_i4_f64(p4, s4, 9, 200, x)
    assert np.allclose(oracle.dequant_f64(p4, s4, 9, 200, 4) @ x.astype(np.float64), y4,
                       rtol=1e-12)


def test_moe_layer_token_rows_match_the_whole_layer():
    # the memory-light form used at full size agrees with the whole-layer
    # oracle (itself pinned by the closed forms above) on every row
    E, F, D, T, k = 5, 64, 192, 6, 3
    mats = []
    for n, (O, I) in enumerate(((F, D), (F, D), (D, F))):
        ps, ss = [], []
        for e in range(E):
            s, c, _ = oracle.quantize_g64(workloads.generic_weights(O, I, seed=7000 + 10 * n + e))
            ps.append(oracle.pack_i3(c))
            ss.append(s)
        mats.append((np.stack(ps), np.stack(ss), 3))
    X = workloads.generic_matrix(T, D, seed=71)
    logits = workloads.rng_for("generic", 72, T, E).random((T, E)).astype(np.float32)
    ref, bound = oracle.moe_layer_f64(X, logits, k, *mats)

    def expert(e):
        return tuple((m[0][e], m[1][e], m[2]) for m in mats)

    rows = [4, 0, 5]
    out, b2 = oracle.moe_layer_f64_tokens(X, logits, k, expert, rows)
    assert np.allclose(out, ref[rows], rtol=1e-12, atol=1e-300)
    assert np.allclose(b2, bound[rows], rtol=1e-12, atol=1e-300)
