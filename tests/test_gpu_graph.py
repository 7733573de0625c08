"""Graph capture: each entry point is captured in a HIP graph
(torch.cuda.CUDAGraph) and replayed three times.  Before each replay new
input values are written into the captured input buffers (eager work, then
a synchronization), and after it every output is compared bit for bit with
an eager call of the same entry point on the same inputs.  The library
enqueues only kernels (no memset, no allocation), so a replay must repeat the
eager work exactly, data-dependent routing included."""
import numpy as np
import pytest
import torch

import dequant_matmul_int3_amd as qt
import workloads
from tests.gpu_util import DEV, bits, host, say

pytestmark = pytest.mark.gpu


def graph_matches_eager(tag, refill, run, outs_graph, outs_eager, replays=3):
    """refill(r): new values into the captured inputs; run(outs): enqueue the
    entry point writing into outs (a list of tensors)."""
    refill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        run(outs_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(outs_graph)
    for r in range(replays):
        refill(r + 1)
        torch.cuda.synchronize()
        g.replay()
        run(outs_eager)
        torch.cuda.synchronize()
        for a, b in zip(outs_graph, outs_eager):
            assert np.array_equal(bits(host(a)), bits(host(b))), f"{tag}: replay {r} differs"
    say(f"graph {tag}: {replays} replays equal the eager calls")


def filler(*pairs):
    """refill(r) writing seeded values into each (tensor, scale) pair."""
    def refill(r):
        for n, (t, scale) in enumerate(pairs):
            g = torch.Generator().manual_seed(1000 * r + n)
            t.copy_((torch.randn(t.shape, generator=g) * scale).to(t.dtype))
    return refill


def packed_weights(O, I, seed, bits_=3):
    W = torch.from_numpy(workloads.generic_weights(O, I, seed=seed)).to(DEV)
    if bits_ == 3:
        s, c, _ = qt.qt_quantize_g64(W, want_grid_idx=False)
        return qt.qt_pack_i3(c), s
    s, c, _ = qt.qt_quantize_g64_i4(W, want_grid_idx=False)
    return qt.qt_pack_i4(c), s


def test_graph_decode_gemv():
    O, I = 2048, 7168
    p, s = packed_weights(O, I, 1)
    x = torch.empty(I, dtype=torch.float32, device=DEV)
    yg, ye = (torch.empty(O, dtype=torch.float32, device=DEV) for _ in range(2))
    graph_matches_eager("decode GEMV 2048x7168", filler((x, 1.0)),
                        lambda o: qt.qt_matvec_i3(p, s, O, I, x, o[0]), [yg], [ye])


@pytest.mark.parametrize("B,xt", [(4, torch.float32), (64, torch.bfloat16)])
def test_graph_matmul(B, xt):
    O, I = 300, 1000  # ragged tiles; bf16 at B = 64 takes the matrix-core path
    p, s = packed_weights(O, I, 2)
    X = torch.empty((B, I), dtype=xt, device=DEV)
    Yg, Ye = (torch.empty((B, O), dtype=torch.float32, device=DEV) for _ in range(2))
    graph_matches_eager(f"matmul B={B} {xt}", filler((X, 1.0)),
                        lambda o: qt.qt_matmul_i3(p, s, O, I, X, o[0]), [Yg], [Ye])


def test_graph_grouped():
    E, O, I, T = 5, 256, 640, 6
    ps, ss = zip(*(packed_weights(O, I, 10 + e) for e in range(E)))
    pk, sc = torch.stack(ps), torch.stack(ss)
    offs = torch.tensor([0, 3, 3, 7, 8, 11], dtype=torch.int32, device=DEV)
    rows = torch.tensor([0, 2, 5, 1, 2, 3, 4, 0, 1, 3, 5], dtype=torch.int32, device=DEV)
    P = rows.numel()
    X = torch.empty((T, I), dtype=torch.float32, device=DEV)
    Yg, Ye = (torch.empty((P, O), dtype=torch.float32, device=DEV) for _ in range(2))
    graph_matches_eager("grouped MoE GEMV", filler((X, 1.0)),
                        lambda o: qt.qt_matvec_i3_grouped(pk, sc, E, O, I, X, offs, P,
                                                          pair_row=rows, Y=o[0]), [Yg], [Ye])


def test_graph_quantize_search_and_pack():
    O, I = 96, 700
    W = torch.empty((O, I), dtype=torch.float32, device=DEV)
    d = torch.empty(I, dtype=torch.float32, device=DEV)

    def refill(r):
        filler((W, 0.02))(r)
        g = torch.Generator().manual_seed(77 + r)
        d.copy_(torch.exp(torch.randn(I, generator=g)))

    G = qt.qt_groups(I)

    def outs():
        return [torch.empty((O, G), dtype=torch.float32, device=DEV),
                torch.empty((O, I), dtype=torch.int8, device=DEV),
                torch.empty((O, G), dtype=torch.uint8, device=DEV),
                torch.empty(qt.qt_packed_bytes(O, I), dtype=torch.uint8, device=DEV)]

    def run(o):
        qt.qt_quantize_g64(W, d, 64, 0.5, 1.0, scales=o[0], codes=o[1], grid_idx=o[2])
        qt.qt_pack_i3(o[1], o[3])

    graph_matches_eager("weighted search + pack", refill, run, outs(), outs())


def test_graph_hessians():
    T, I = 300, 640  # several token slabs: the diagonal's workspace is used
    X = torch.empty((T, I), dtype=torch.float32, device=DEV)
    Xb = torch.empty((T, I), dtype=torch.bfloat16, device=DEV)
    wd = torch.empty(max(1, qt.qt_hessian_workspace_bytes(T, I)), dtype=torch.uint8, device=DEV)
    wf = torch.empty(qt.qt_hessian_full_workspace_bytes(T, I, qt.QT_BF16), dtype=torch.uint8,
                     device=DEV)

    def outs():
        return [torch.empty(I, dtype=torch.float32, device=DEV),
                torch.empty((I, I), dtype=torch.float32, device=DEV)]

    def run(o):
        qt.qt_hessian_diag(X, o[0], workspace=wd)
        qt.qt_hessian_full(Xb, o[1], workspace=wf)

    graph_matches_eager("Hessian diagonal + full (bf16)", filler((X, 1.0), (Xb, 1.0)), run,
                        outs(), outs())


def test_graph_moe_layer():
    E, F, D, T, k = 8, 256, 512, 9, 2
    gate = (*packed_weights_stack(E, F, D, 100), 3)
    up = (*packed_weights_stack(E, F, D, 200), 3)
    down = (*packed_weights_stack(E, D, F, 300), 3)
    X = torch.empty((T, D), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ws = torch.empty(qt.qt_moe_layer_workspace_bytes(T, k, E, D, F), dtype=torch.uint8,
                     device=DEV)
    Og, Oe = (torch.empty((T, D), dtype=torch.float32, device=DEV) for _ in range(2))
    # new logits before every replay: the routing changes inside the graph
    graph_matches_eager("MoE expert layer", filler((X, 1.0), (logits, 1.0)),
                        lambda o: qt.qt_moe_layer(X, logits, k, gate, up, down, out=o[0],
                                                  workspace=ws), [Og], [Oe])


def packed_weights_stack(E, O, I, seed):
    ps, ss = zip(*(packed_weights(O, I, seed + e) for e in range(E)))
    return torch.stack(ps), torch.stack(ss)
