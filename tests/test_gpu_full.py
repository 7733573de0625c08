"""Parity at the full workload sizes, in the launch configurations bench.py
times, on sampled outputs the oracle computes one by one.

Decode (W[2048x7168] and the 7200 tail variant) is compared in full in
test_gpu_parity.py; here: the prefill GEMM, the 128-expert MoE grouped GEMV
and the weighted scale search with its Hessian diagonal.
"""
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


def test_prefill_gemm_full_size_sampled():
    O, I = workloads.PREFILL_SHAPE
    G = qt.qt_groups(I)
    say(f"prefill: quantize+pack W[{O}x{I}] in 1024-row slabs on the GPU")
    pk = torch.empty(qt.qt_packed_bytes(O, I), dtype=torch.uint8, device="cuda:0")
    sc = torch.empty((O, G), dtype=torch.float32, device="cuda:0")
    codes_dev = torch.empty((O, I), dtype=torch.int8, device="cuda:0")
    for s in range(O // 1024):
        w = dev(workloads.prefill_w([s]))
        qt.qt_quantize_g64(w, scales=sc[s * 1024:(s + 1) * 1024],
                           codes=codes_dev[s * 1024:(s + 1) * 1024], want_grid_idx=False)
    qt.qt_pack_i3(codes_dev, pk)
    Xb = workloads.prefill_x()
    B = Xb.shape[0]
    say(f"prefill: GEMM B={B}")
    Y = host(qt.qt_matmul_i3(pk, sc, O, I, dev_bf16(Xb)))
    Xf = workloads.bf16_bits_to_f32(Xb)
    rng = workloads.rng_for("generic", 9001)
    slabs = rng.choice(O // 1024, size=3, replace=False)
    pk_h, sc_h = host(pk), host(sc)
    worst = 0.0
    for s in slabs:
        Wslab = workloads.prefill_w([int(s)])
        so, co, _ = oracle.quantize_g64(Wslab)
        rows = np.arange(s * 1024, (s + 1) * 1024)
        assert np.array_equal(bits(sc_h[rows]), bits(so)), "scales differ"
        po = oracle.pack_i3(co)
        assert np.array_equal(pk_h.reshape(O, G * 24)[rows].reshape(-1), po), "packed differ"
        # sampled outputs of this slab
        t_idx = rng.integers(0, B, size=96)
        o_loc = rng.integers(0, 1024, size=96)
        yr, ar = oracle.matmul_f64_sampled(po, so, 1024, I, Xf, t_idx, o_loc)
        err = componentwise_err(Y[t_idx, s * 1024 + o_loc], yr, ar)
        worst = max(worst, err)
    say(f"  sampled componentwise err {worst:.3e}")
    assert worst <= TOL_MFMA


def test_moe_grouped_full_size_sampled():
    E = workloads.MOE_EXPERTS
    (Ou, Iu), (Od, Id) = workloads.MOE_UP_SHAPE, workloads.MOE_DOWN_SHAPE
    Gu, Gd = qt.qt_groups(Iu), qt.qt_groups(Id)
    d0 = "cuda:0"
    pu = torch.empty((E, qt.qt_packed_bytes(Ou, Iu)), dtype=torch.uint8, device=d0)
    su = torch.empty((E, Ou, Gu), dtype=torch.float32, device=d0)
    pdn = torch.empty((E, qt.qt_packed_bytes(Od, Id)), dtype=torch.uint8, device=d0)
    sdn = torch.empty((E, Od, Gd), dtype=torch.float32, device=d0)
    for which, pk, sc in (("up", pu, su), ("down", pdn, sdn)):
        say(f"moe: quantize+pack 128 {which} matrices on the GPU")
        for e0 in range(0, E, 16):
            mats = workloads.moe_experts_parallel(which, range(e0, e0 + 16), workers=16)
            for j, m in enumerate(mats):
                s_, c_, _ = qt.qt_quantize_g64(dev(m), want_grid_idx=False)
                sc[e0 + j].copy_(s_)
                qt.qt_pack_i3(c_, pk[e0 + j])
            torch.cuda.synchronize()
    Xm, top = workloads.moe_tokens()
    tok, exp, offs = workloads.route_pairs(top, E)
    P = tok.size
    say(f"moe: grouped up P={P}, experts hit {int(np.count_nonzero(np.diff(offs)))}")
    h = qt.qt_matvec_i3_grouped(pu, su, E, Ou, Iu, dev(Xm), dev(offs), P, pair_row=dev(tok))
    H = workloads.generic_matrix(P, Id, seed=4321)
    say("moe: grouped down on an independent input")
    yd = qt.qt_matvec_i3_grouped(pdn, sdn, E, Od, Id, dev(H), dev(offs), P)
    h, yd = host(h), host(yd)
    rng = workloads.rng_for("generic", 9002)
    sample = rng.choice(P, size=16, replace=False)
    worst_u = worst_d = 0.0
    for p in sample:
        e, t = int(exp[p]), int(tok[p])
        so, co, _ = oracle.quantize_g64(workloads.moe_expert(e, "up"))
        po = oracle.pack_i3(co)
        assert np.array_equal(host(pu[e]), po) and np.array_equal(bits(host(su[e])), bits(so))
        yr, ar = oracle.matvec_f64(po, so, Ou, Iu, Xm[t])
        worst_u = max(worst_u, componentwise_err(h[p], yr, ar))
        so, co, _ = oracle.quantize_g64(workloads.moe_expert(e, "down"))
        po = oracle.pack_i3(co)
        yr, ar = oracle.matvec_f64(po, so, Od, Id, H[p])
        worst_d = max(worst_d, componentwise_err(yd[p], yr, ar))
    say(f"  sampled componentwise err up {worst_u:.3e} down {worst_d:.3e}")
    assert worst_u <= TOL_F32 and worst_d <= TOL_F32


def test_search_and_hessian_full_size_sampled():
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
    rng = workloads.rng_for("generic", 9003)
    rows = np.sort(rng.choice(O, size=12, replace=False))
    so, co, ko = oracle.quantize_g64(W[rows], d, 64, 0.5, 1.0)
    assert np.array_equal(bits(s[rows]), bits(so)), "scales differ"
    assert np.array_equal(c[rows], co), "codes differ"
    assert np.array_equal(k[rows], ko), "grid indices differ"
    say(f"  {rows.size} sampled rows bit-exact; grid index histogram head "
        f"{np.bincount(k.reshape(-1), minlength=64)[:4]}")
    say(f"search: W[{O}x{I}] two-stage signed 64/32 weighted search on the GPU")
    s2, c2 = qt.qt_quantize_g64_signed(dev(W), dev(d), 64, 32, 0.5, 1.0)
    s2, c2 = host(s2), host(c2)
    rows = np.sort(rng.choice(O, size=6, replace=False))
    so2, co2 = oracle.quantize_g64_signed(W[rows], d, 64, 32, 0.5, 1.0)
    assert np.array_equal(bits(s2[rows]), bits(so2)), "signed scales differ"
    assert np.array_equal(c2[rows], co2), "signed codes differ"
    say(f"  {rows.size} sampled rows bit-exact; negative scales {np.mean(s2 < 0):.3f}")
