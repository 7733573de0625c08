"""The MoE expert layer (routing, gate/up, SwiGLU, down and combine
launches) against the oracle's f64 layer: every output
within 1e-5 of the error budget the oracle derives from the grouped
multiply's tolerance."""
import numpy as np
import pytest
import torch

import dequant_matmul_int3_amd as qt
import oracle
import workloads
from tests.gpu_util import bits as fbits, dev, host, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def experts(E, F, D, seed, bits):
    out = []
    for n, ((O, I), b) in enumerate((((F, D), bits[0]), ((F, D), bits[1]), ((D, F), bits[2]))):
        ps, ss = [], []
        for e in range(E):
            W = workloads.generic_weights(O, I, seed=seed * 1000 + 100 * n + e)
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


def run_gpu(X, logits, k, gate, up, down):
    g = tuple(dev(a) if isinstance(a, np.ndarray) else a for a in gate)
    u = tuple(dev(a) if isinstance(a, np.ndarray) else a for a in up)
    d = tuple(dev(a) if isinstance(a, np.ndarray) else a for a in down)
    return host(qt.qt_moe_layer(dev(X), dev(logits), k, g, u, d))


def check(X, logits, k, gate, up, down, tag):
    T, D = X.shape
    say(f"moe layer {tag} T={T} D={D} E={logits.shape[1]} k={k}")
    out = run_gpu(X, logits, k, gate, up, down)
    ref, bound = oracle.moe_layer_f64(X, logits, k, gate, up, down)
    err = np.max(np.abs(out - ref) / bound)
    say(f"  max error / budget {err:.3e}")
    assert err <= TOL
    return out


@pytest.mark.parametrize("scheme", [(3, 3, 3), (4, 3, 4), (4, 4, 4), (3, 4, 3)])
def test_moe_layer_schemes(scheme):
    E, F, D, T, k = 6, 128, 256, 5, 2
    gate, up, down = experts(E, F, D, 1, scheme)
    X = workloads.generic_matrix(T, D, seed=2)
    logits = workloads.rng_for("generic", 900, T, E).random((T, E)).astype(np.float32)
    check(X, logits, k, gate, up, down, f"bits {scheme}")


@pytest.mark.parametrize("E,F,D,T,k", [(16, 256, 512, 12, 4), (8, 128, 128, 33, 8),
                                       (3, 384, 256, 1, 1), (5, 128, 384, 7, 5)])
def test_moe_layer_shapes(E, F, D, T, k):
    gate, up, down = experts(E, F, D, E + T, (3, 3, 3))
    X = workloads.generic_matrix(T, D, seed=T)
    logits = workloads.rng_for("generic", 901, T, E).random((T, E)).astype(np.float32)
    out1 = check(X, logits, k, gate, up, down, "shape")
    out2 = run_gpu(X, logits, k, gate, up, down)
    assert np.array_equal(fbits(out1), fbits(out2)), "not deterministic"


@pytest.mark.parametrize("E,T,k", [(200, 70, 3),    # 17-32 experts per 16 lanes, 32 tokens a pass
                                   (300, 40, 2),    # 33-64 experts per 16 lanes, 16 tokens a pass
                                   (512, 17, 32),   # the largest E and k
                                   (8, 700, 8),     # 5600 pairs: the pair table past its LDS size
                                   (128, 129, 8)])  # two passes of 64 tokens and one token more
def test_moe_layer_routing_sizes(E, T, k):
    # every routing variant over several passes of tokens; ranks of a token
    # among the earlier tokens of its expert cross pass boundaries
    F, D = 128, 128
    gate, up, down = experts(E, F, D, E + T, (3, 3, 3))
    X = workloads.generic_matrix(T, D, seed=T + 1)
    logits = workloads.rng_for("generic", 902, T, E).random((T, E)).astype(np.float32)
    out1 = check(X, logits, k, gate, up, down, "routing sizes")
    out2 = run_gpu(X, logits, k, gate, up, down)
    assert np.array_equal(fbits(out1), fbits(out2)), "not deterministic"


@pytest.mark.parametrize("E,T,k", [(1, 3, 1),      # one expert: every pair on it
                                   (4, 70, 4),     # k = E: every token picks every expert
                                   (2, 64, 1)])    # exactly one pass of 64 tokens
def test_moe_layer_routing_degenerate(E, T, k):
    F, D = 128, 128
    gate, up, down = experts(E, F, D, 300 + E + T, (3, 3, 3))
    X = workloads.generic_matrix(T, D, seed=T + 7)
    logits = workloads.rng_for("generic", 903, T, E).random((T, E)).astype(np.float32)
    check(X, logits, k, gate, up, down, "degenerate routing")


def test_moe_layer_routing_ties_and_idle_experts():
    # tied logits pick the lower expert first; experts nobody picks are idle
    E, F, D, T, k = 8, 128, 128, 4, 3
    gate, up, down = experts(E, F, D, 5, (3, 3, 3))
    X = workloads.generic_matrix(T, D, seed=6)
    logits = np.zeros((T, E), np.float32)
    logits[0, [2, 5, 6]] = 1.0          # a three-way tie at the top
    logits[1, [1, 2]] = [0.5, 0.5]      # tie for the first two, then index order
    logits[2] = np.arange(E, dtype=np.float32)[::-1]
    logits[3, 7] = 2.0
    check(X, logits, k, gate, up, down, "ties")


def test_moe_layer_full_size_sampled():
    # the benched shape: 128 experts of gate/up [2048x7168] and down
    # [7168x2048], int3-g64 everywhere, 32 tokens, top-8 of uniform logits.
    # Every expert's bytes and scales are checked against the oracle's; six
    # tokens' outputs against the oracle's f64 layer within the error budget.
    from concurrent.futures import ThreadPoolExecutor
    import os
    E, T, k = workloads.MOE_EXPERTS, workloads.MOE_TOKENS, workloads.MOE_TOPK
    F, D = workloads.MOE_UP_SHAPE
    threads = min(16, os.cpu_count() or 1)
    X, _ = workloads.moe_tokens()
    logits = workloads.moe_logits().astype(np.float32)
    rng = workloads.rng_for("generic", 9004)
    tokens = sorted(int(t) for t in rng.choice(T, size=6, replace=False))
    used = set(int(e) for e in oracle.moe_route(logits, k)[0][tokens].reshape(-1))
    shapes = {"gate": (F, D), "up": (F, D), "down": (D, F)}
    dev_mats, keep = {}, {e: {} for e in used}

    def oq(m):
        s, c, _ = oracle.quantize_g64(m)
        return s, oracle.pack_i3(c)

    with ThreadPoolExecutor(threads) as ex:
        for proj in ("gate", "up", "down"):
            O, I = shapes[proj]
            pk = torch.empty((E, qt.qt_packed_bytes(O, I)), dtype=torch.uint8, device="cuda:0")
            sc = torch.empty((E, O, qt.qt_groups(I)), dtype=torch.float32, device="cuda:0")
            say(f"moe layer full size: quantize+pack 128 {proj} matrices (GPU and oracle)")
            for e0 in range(0, E, 16):
                mats = workloads.moe_experts_parallel(proj, range(e0, e0 + 16), workers=16)
                for j, m in enumerate(mats):
                    s_, c_, _ = qt.qt_quantize_g64(dev(m), want_grid_idx=False)
                    sc[e0 + j].copy_(s_)
                    qt.qt_pack_i3(c_, pk[e0 + j])
                refs = list(ex.map(oq, mats))
                del mats
                for j, (so, po) in enumerate(refs):
                    e = e0 + j
                    assert np.array_equal(fbits(host(sc[e])), fbits(so)), f"{proj} scales, expert {e}"
                    assert np.array_equal(host(pk[e]), po), f"{proj} bytes, expert {e}"
                    if e in used:
                        keep[e][proj] = (po, so, 3)
            dev_mats[proj] = (pk, sc, 3)
    say(f"moe layer full size: E={E} T={T} k={k}, sampled tokens {tokens}")
    out = host(qt.qt_moe_layer(dev(X), dev(logits), k, dev_mats["gate"], dev_mats["up"],
                               dev_mats["down"]))
    out2 = host(qt.qt_moe_layer(dev(X), dev(logits), k, dev_mats["gate"], dev_mats["up"],
                                dev_mats["down"]))
    assert np.array_equal(fbits(out), fbits(out2)), "not deterministic"

    def expert(e):
        return keep[e]["gate"], keep[e]["up"], keep[e]["down"]

    ref, bound = oracle.moe_layer_f64_tokens(X, logits, k, expert, tokens)
    err = np.max(np.abs(out[tokens] - ref) / bound)
    say(f"  max error / budget {err:.3e} over {len(tokens)} tokens x {D} outputs")
    assert err <= TOL
