"""Parity at the full workload sizes, in the launch configurations bench.py
times.

Bit-exact over the whole of each configuration: every prefill slab's scales
and packed bytes, every MoE expert's up and down matrices, every row of the
weighted and the signed scale search (scales, codes, grid indices).  The f32
products are compared on outputs the oracle computes one by one (all 256
(token, expert) pairs of the MoE step for up and down, 16 outputs of every
prefill slab).  The oracle runs on a pool of host threads: each call is a C
function reached through ctypes, which releases the interpreter lock.

The full Hessian of the GPTQ leg (bf16 X[8192x17408]) is compared on a
64 x 64 block of H whose rows and columns straddle its 256-wide tile borders.

Decode (W[2048x7168] and the 7200 tail variant) is compared in full in
test_gpu_parity.py.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import dequant_matmul_int3_amd as qt
import oracle
import workloads
from tests.gpu_util import bits, dev, dev_bf16, host, say
from tests.parity import componentwise_err

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_MFMA = 2e-3
THREADS = min(16, os.cpu_count() or 1)


def oracle_quant_pack(W):
    so, co, _ = oracle.quantize_g64(W)
    return so, oracle.pack_i3(co)


def test_prefill_gemm_full_size():
    O, I = workloads.PREFILL_SHAPE
    G = qt.qt_groups(I)
    nslab = O // 1024
    say(f"prefill: quantize+pack W[{O}x{I}] in {nslab} slabs of 1024 rows on the GPU")
    pk = torch.empty(qt.qt_packed_bytes(O, I), dtype=torch.uint8, device="cuda:0")
    sc = torch.empty((O, G), dtype=torch.float32, device="cuda:0")
    codes_dev = torch.empty((O, I), dtype=torch.int8, device="cuda:0")
    slabs = []
    for s in range(nslab):
        w = workloads.prefill_w([s])
        slabs.append(w)
        qt.qt_quantize_g64(dev(w), scales=sc[s * 1024:(s + 1) * 1024],
                           codes=codes_dev[s * 1024:(s + 1) * 1024], want_grid_idx=False)
    qt.qt_pack_i3(codes_dev, pk)
    del codes_dev
    Xb = workloads.prefill_x()
    B = Xb.shape[0]
    say(f"prefill: GEMM B={B}")
    Y = host(qt.qt_matmul_i3(pk, sc, O, I, dev_bf16(Xb)))
    Xf = workloads.bf16_bits_to_f32(Xb)
    pk_h, sc_h = host(pk).reshape(O, G * 24), host(sc)
    say(f"prefill: oracle quantize+pack of all {nslab} slabs on {THREADS} threads")
    with ThreadPoolExecutor(THREADS) as ex:
        ref = list(ex.map(oracle_quant_pack, slabs))
    del slabs
    for s, (so, po) in enumerate(ref):
        rows = slice(s * 1024, (s + 1) * 1024)
        assert np.array_equal(bits(sc_h[rows]), bits(so)), f"scales differ in slab {s}"
        assert np.array_equal(pk_h[rows].reshape(-1), po), f"packed bytes differ in slab {s}"
    # 16 sampled outputs of every slab against the f64 oracle
    rng = workloads.rng_for("generic", 9001)

    def slab_err(s):
        so, po = ref[s]
        t_idx = rng_t[s]
        o_loc = rng_o[s]
        yr, ar = oracle.matmul_f64_sampled(po, so, 1024, I, Xf, t_idx, o_loc)
        return componentwise_err(Y[t_idx, s * 1024 + o_loc], yr, ar)

    rng_t = [rng.integers(0, B, size=16) for _ in range(nslab)]
    rng_o = [rng.integers(0, 1024, size=16) for _ in range(nslab)]
    with ThreadPoolExecutor(THREADS) as ex:
        worst = max(ex.map(slab_err, range(nslab)))
    say(f"  all {nslab} slabs bit-exact; {16 * nslab} sampled outputs, componentwise err "
        f"{worst:.3e}")
    assert worst <= TOL_MFMA
    # the kernel's own bound (exact products, f32 sums): see test_gpu_parity
    assert worst <= (64 + G + 2) * 2.0 ** -24


def test_moe_grouped_full_size():
    E = workloads.MOE_EXPERTS
    (Ou, Iu), (Od, Id) = workloads.MOE_UP_SHAPE, workloads.MOE_DOWN_SHAPE
    Gu, Gd = qt.qt_groups(Iu), qt.qt_groups(Id)
    d0 = "cuda:0"
    Xm, top = workloads.moe_tokens()
    tok, exp, offs = workloads.route_pairs(top, E)
    P = tok.size
    hit = set(int(e) for e in np.unique(exp))
    pu = torch.empty((E, qt.qt_packed_bytes(Ou, Iu)), dtype=torch.uint8, device=d0)
    su = torch.empty((E, Ou, Gu), dtype=torch.float32, device=d0)
    pdn = torch.empty((E, qt.qt_packed_bytes(Od, Id)), dtype=torch.uint8, device=d0)
    sdn = torch.empty((E, Od, Gd), dtype=torch.float32, device=d0)
    ref = {"up": {}, "down": {}}  # the oracle's bytes of the experts that pairs hit
    with ThreadPoolExecutor(THREADS) as ex:
        for which, pk, sc in (("up", pu, su), ("down", pdn, sdn)):
            say(f"moe: quantize+pack 128 {which} matrices on the GPU and in the oracle")
            for e0 in range(0, E, 16):
                mats = workloads.moe_experts_parallel(which, range(e0, e0 + 16), workers=16)
                for j, m in enumerate(mats):
                    s_, c_, _ = qt.qt_quantize_g64(dev(m), want_grid_idx=False)
                    sc[e0 + j].copy_(s_)
                    qt.qt_pack_i3(c_, pk[e0 + j])
                refs = list(ex.map(oracle_quant_pack, mats))
                del mats
                for j, (so, po) in enumerate(refs):
                    e = e0 + j
                    assert np.array_equal(bits(host(sc[e])), bits(so)), f"{which} scales differ, expert {e}"
                    assert np.array_equal(host(pk[e]), po), f"{which} packed bytes differ, expert {e}"
                    if e in hit:
                        ref[which][e] = (so, po)
    say(f"moe: all 128 experts bit-exact (up and down); grouped up P={P}, "
        f"experts hit {len(hit)}")
    h = host(qt.qt_matvec_i3_grouped(pu, su, E, Ou, Iu, dev(Xm), dev(offs), P, pair_row=dev(tok)))
    H = workloads.generic_matrix(P, Id, seed=4321)
    say("moe: grouped down on an independent input")
    yd = host(qt.qt_matvec_i3_grouped(pdn, sdn, E, Od, Id, dev(H), dev(offs), P))

    def pair_err(p):
        e, t = int(exp[p]), int(tok[p])
        so, po = ref["up"][e]
        yr, ar = oracle.matvec_f64(po, so, Ou, Iu, Xm[t])
        eu = componentwise_err(h[p], yr, ar)
        so, po = ref["down"][e]
        yr, ar = oracle.matvec_f64(po, so, Od, Id, H[p])
        return eu, componentwise_err(yd[p], yr, ar)

    with ThreadPoolExecutor(THREADS) as ex:
        errs = list(ex.map(pair_err, range(P)))
    worst_u = max(e[0] for e in errs)
    worst_d = max(e[1] for e in errs)
    say(f"  all {P} pairs: componentwise err up {worst_u:.3e} down {worst_d:.3e}")
    assert worst_u <= TOL_F32 and worst_d <= TOL_F32


def test_search_and_hessian_full_size():
    O, I = workloads.SEARCH_SHAPE
    say(f"search: X[{workloads.SEARCH_TOKENS}x{I}] Hessian diagonal")
    X = workloads.search_x()
    Xd = dev(X)
    d_gpu = host(qt.qt_hessian_diag(Xd))
    del Xd
    d_ref = oracle.hessian_diag(X)
    del X
    rel = np.max(np.abs(d_gpu - d_ref) / d_ref)
    say(f"  hessian max relative err {rel:.3e}")
    assert rel <= 1e-5
    # the same importance array feeds both sides of the bit-exact search
    d = d_ref.astype(np.float32)
    say(f"search: W[{O}x{I}] 64-point weighted grid on the GPU")
    W = workloads.search_w()
    s, c, k = qt.qt_quantize_g64(dev(W), dev(d), 64, 0.5, 1.0)
    s, c, k = host(s), host(c), host(k)
    slabs = [slice(r, min(r + 64, O)) for r in range(0, O, 64)]
    say(f"search: oracle over all {O} rows on {THREADS} threads")

    def check(rows):
        so, co, ko = oracle.quantize_g64(W[rows], d, 64, 0.5, 1.0)
        return (np.array_equal(bits(s[rows]), bits(so)), np.array_equal(c[rows], co),
                np.array_equal(k[rows], ko))

    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(check, slabs))
    for i, (a, b, g) in enumerate(res):
        assert a, f"scales differ in rows {slabs[i]}"
        assert b, f"codes differ in rows {slabs[i]}"
        assert g, f"grid indices differ in rows {slabs[i]}"
    say(f"  all {O} rows bit-exact; grid index histogram head "
        f"{np.bincount(k.reshape(-1), minlength=64)[:4]}")
    del c
    say(f"search: W[{O}x{I}] two-stage signed 64/32 weighted search on the GPU")
    s2, c2 = qt.qt_quantize_g64_signed(dev(W), dev(d), 64, 32, 0.5, 1.0)
    s2, c2 = host(s2), host(c2)

    def check2(rows):
        so2, co2 = oracle.quantize_g64_signed(W[rows], d, 64, 32, 0.5, 1.0)
        return np.array_equal(bits(s2[rows]), bits(so2)), np.array_equal(c2[rows], co2)

    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(check2, slabs))
    for i, (a, b) in enumerate(res):
        assert a, f"signed scales differ in rows {slabs[i]}"
        assert b, f"signed codes differ in rows {slabs[i]}"
    say(f"  all {O} rows bit-exact; negative scales {np.mean(s2 < 0):.3f}")


def test_hessian_full_full_size():
    # H = X^T X of the GPTQ leg's bf16 X[8192x17408]: the oracle's Hessian of
    # 64 chosen columns is the 64 x 64 block of H on those rows and columns
    I = workloads.SEARCH_SHAPE[1]
    say(f"full Hessian: bf16 X[{workloads.SEARCH_TOKENS}x{I}]")
    Xb = workloads.bf16_bits_rne(workloads.search_x())
    Hd = qt.qt_hessian_full(dev_bf16(Xb))
    edges = [0, 1, 255, 256, 257, 511, 512, 8191, 8192, 8447, 8448, 17151, 17152, 17406, 17407]
    rng = np.random.default_rng(17408)
    rest = rng.choice(np.setdiff1d(np.arange(I), edges), 64 - len(edges), replace=False)
    cols = np.sort(np.concatenate([edges, rest]))
    idx = torch.from_numpy(cols).to(Hd.device)
    Hs = host(Hd.index_select(0, idx).index_select(1, idx))
    del Hd
    Xf = workloads.bf16_bits_to_f32(np.ascontiguousarray(Xb[:, cols]))
    del Xb
    Href = oracle.hessian_full(Xf)
    A = np.abs(Xf.astype(np.float64))
    bound = A.T @ A
    err = np.abs(Hs.astype(np.float64) - Href) / np.maximum(bound, 1e-300)
    say(f"  64 x 64 block: max componentwise err {err.max():.3e}")
    assert err.max() <= 2e-5
    assert np.array_equal(bits(Hs), bits(np.ascontiguousarray(Hs.T))), "not exactly symmetric"
