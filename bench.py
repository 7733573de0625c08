"""Benchmark of the int3-g64 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs all|gemv|LEG[,LEG...]]

Headline (one JSON line on stdout): the decode GEMV, W[2048x7168] int3-g64
with f32 scales times x[7168] f32, batch 1.  A step is one dequantize-multiply
of the whole matrix; consecutive steps read 64 distinct copies of the packed
weights (64 x 6.46 MB = 413 MB, more than the 256 MB Infinity Cache), so every
step streams its weights from HBM.  value = algorithmic bytes per step
(packed weights + scales + x + y = 6,459,392 B) x steps / elapsed time.

The other rows of the hot path are timed as "legs" on their own workloads:
the Hessian diagonal and the weighted scale search (W[5120x17408],
X[8192x17408]), plain quantize + pack at the decode shape, the grouped MoE
GEMV (128 experts, 32 tokens, top-8) and the bf16 MFMA prefill GEMM
(X[512x7168] x W[18432x7168]); grouped int4: the decode GEMV with int4
weights and the MoE step with every projection at int4 and with up at int3
(the per-projection mix).  Every input is seeded synthetic data
(workloads.py) resident on the GPU before its timed region starts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
# Vector ALU: the published fp32 vector peak, 157.3 TFLOP/s, counts an FMA as
# two operations: 78.65 T lane-operations/s.  (Single-issue non-packed f32
# instructions measure 64 lanes/clock/CU = 39.3 T at 2.4 GHz; round-to-integer
# issues beside them, so an op count can exceed that figure.)
VALU_PEAK_TOPS = 157.3 / 2
N_COPIES = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--legs", default="all",
                    help="all, gemv (headline only) or a comma list of: " + ",".join(LEG_NAMES))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib", action="store_true",
                    help="also run a 256 MiB device copy (reference for HBM traffic counters)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sha_of(*rel):
    h = hashlib.sha256()
    for r in rel:
        with open(os.path.join(ROOT, r), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(name, bytes_alg):
    """Measured HBM bytes per launch from profiles/<name>_traffic.json, if the
    kernel source is unchanged since the counters were taken; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha") != sha_of(*rec.get("sources", [])):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, n, torch, warmup=2):
    """Average time per fn() call over n back-to-back calls, from a pair of
    events on the current stream (the stream the kernels run on), after
    `warmup` untimed calls."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(n):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    return total_ms / n


def graph_ms(fn, n_copies, warmup, steps, torch):
    """Per-call time of fn(j), j = 0..n_copies-1, captured once in a HIP
    graph and replayed until `steps` calls are timed (so that host-side call
    overhead does not pace the GPU)."""
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        for j in range(n_copies):
            fn(j)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for j in range(n_copies):
            fn(j)
    for _ in range(max(1, -(-warmup // n_copies))):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // n_copies))
    return time_launches(lambda i: graph.replay(), reps, torch) / n_copies, reps * n_copies


def per_launch_ms(fn, n, torch):
    """Mean and median of single fn() calls, each bracketed by its own events."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(st)
        fn(i)
        b.record(st)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.mean(d)), float(np.median(d))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_matmul_int3_amd as qt
    import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    legs = {}

    # ------------------------------------------------------------ decode GEMV
    W, x = workloads.decode()
    O, I = W.shape
    G = qt.qt_groups(I)
    log(f"decode GEMV {O}x{I}: quantize + pack on the GPU")
    Wd = torch.from_numpy(W).to(dev)
    xd = torch.from_numpy(x).to(dev)
    s, c, _ = qt.qt_quantize_g64(Wd)
    p = qt.qt_pack_i3(c)
    torch.cuda.synchronize()
    packs = torch.empty((N_COPIES, p.numel()), dtype=torch.uint8, device=dev)
    scs = torch.empty((N_COPIES, O, G), dtype=torch.float32, device=dev)
    packs.copy_(p.expand(N_COPIES, -1))
    scs.copy_(s.expand(N_COPIES, -1, -1))
    y = torch.empty(O, dtype=torch.float32, device=dev)
    bytes_step = p.numel() + s.numel() * 4 + I * 4 + O * 4

    def gemv(j):
        qt.qt_matvec_i3(packs[j], scs[j], O, I, xd, y)

    # the launch loop is captured in a HIP graph (one launch per weight copy)
    # so that host-side call overhead does not pace the GPU
    log(f"decode GEMV: capture {N_COPIES} launches, warmup {args.warmup}, timed {args.steps} steps")
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        for j in range(N_COPIES):
            gemv(j)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for j in range(N_COPIES):
            gemv(j)
    reps_w = max(1, -(-args.warmup // N_COPIES))
    reps = max(1, -(-args.steps // N_COPIES))
    steps = reps * N_COPIES
    for _ in range(reps_w):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = time_launches(lambda i: graph.replay(), reps, torch) / N_COPIES
    value = bytes_step / (ms_step * 1e-3) / 1e9
    achieved = value
    # eager single launches bracketed by their own events, for reference
    kmean, kmed = per_launch_ms(lambda i: gemv(i % N_COPIES), 256, torch)
    tr = traffic_for("gemv_decode", bytes_step)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": tr, "kernel": "gemv_batch_kernel<128,16,1,128,f32,vec>",
                "launch_us_mean": round(ms_step * 1e3, 3),
                "eager_event_pair_us_mean": round(kmean * 1e3, 3),
                "bytes_per_launch": bytes_step}
    log(f"  {ms_step * 1e3:.2f} us/launch back-to-back (graph) = {value:.0f} GB/s; "
        f"eager event pair {kmean * 1e3:.2f} us")
    del packs, scs

    if args.calib:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings
        # calibrate the traffic counters of the kernels above
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.legs != "gemv":
        which = set(LEG_NAMES) if args.legs == "all" else set(args.legs.split(","))
        unknown = which - set(LEG_NAMES)
        if unknown:
            raise SystemExit(f"unknown legs {sorted(unknown)}; choose from {LEG_NAMES}")
        legs.update(run_legs(torch, qt, workloads, dev, which, args))

    cpu = cpu_baseline(W, x, args.cpu_seconds, bytes_step)

    line = {
        "metric": "int3-g64 GEMV effective HBM GB/s (% of peak) at I=7168; quantize groups/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode GEMV: W[2048x7168] int3-g64 (f32 scales) x x[7168] f32, "
                               "batch 1, 64 rotating weight copies",
                   "O": O, "I": I, "batch": 1, "rotating_copies": N_COPIES,
                   "bytes_per_step": bytes_step},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": legs,
    }
    if "quantize_search" in legs:
        line["quantize_groups_per_s"] = legs["quantize_search"]["groups_per_s"]
    print(json.dumps(line), flush=True)


LEG_NAMES = ["quant", "search", "moe", "prefill", "int4", "moe_int4", "gptq", "moe_layer"]


def run_legs(torch, qt, workloads, dev, which, args):
    """Time the selected legs: quant (RTN quantize + pack at the decode shape),
    search (Hessian diagonal + weighted scale search), moe (grouped GEMV),
    prefill (bf16 MFMA GEMM), int4 (grouped-int4 quantize, pack and decode
    GEMV), moe_int4 (the MoE step at int4 and with up at int3)."""
    legs = {}
    if "quant" in which:
        quant_leg(torch, qt, workloads, dev, legs)
    if "search" in which:
        search_leg(torch, qt, workloads, dev, legs)
    if "moe" in which or "moe_int4" in which:
        moe_leg(torch, qt, workloads, dev, legs, "moe" in which, "moe_int4" in which)
    if "prefill" in which:
        prefill_leg(torch, qt, workloads, dev, legs)
    if "int4" in which:
        int4_leg(torch, qt, workloads, dev, legs, args)
    if "gptq" in which:
        gptq_leg(torch, qt, workloads, dev, legs)
    if "moe_layer" in which:
        moe_layer_leg(torch, qt, workloads, dev, legs)
    return legs


def moe_layer_leg(torch, qt, workloads, dev, legs):
    # ------------------- MoE expert layer (gate/up/down, routing, combine)
    E, T, k = workloads.MOE_EXPERTS, workloads.MOE_TOKENS, workloads.MOE_TOPK
    (F, D) = workloads.MOE_UP_SHAPE
    log("leg moe_layer: generating and quantizing 128 experts x (gate, up, down)")
    fmt = {3: (qt.qt_packed_bytes, qt.qt_quantize_g64, qt.qt_pack_i3),
           4: (qt.qt_packed_bytes_i4, qt.qt_quantize_g64_i4, qt.qt_pack_i4)}
    need = {("gate", 3), ("up", 3), ("down", 3), ("gate", 4), ("down", 4)}
    shapes = {"gate": (F, D), "up": (F, D), "down": (D, F)}
    store = {}
    for proj, b in need:
        O_, I_ = shapes[proj]
        store[proj, b] = (torch.empty((E, fmt[b][0](O_, I_)), dtype=torch.uint8, device=dev),
                          torch.empty((E, O_, qt.qt_groups(I_)), dtype=torch.float32, device=dev), b)
    for proj in ("gate", "up", "down"):
        bl = sorted(b for (pr, b) in need if pr == proj)
        for e0 in range(0, E, 16):
            mats = workloads.moe_experts_parallel(proj, range(e0, e0 + 16), workers=16)
            for j, m in enumerate(mats):
                md = torch.from_numpy(m).to(dev)
                for b in bl:
                    pk, sc, _ = store[proj, b]
                    s_, c_, _ = fmt[b][1](md, want_grid_idx=False)
                    sc[e0 + j].copy_(s_)
                    fmt[b][2](c_, pk[e0 + j])
            torch.cuda.synchronize()
    Xm, _ = workloads.moe_tokens()
    Xd = torch.from_numpy(Xm).to(dev)
    Ld = torch.from_numpy(workloads.moe_logits().astype(np.float32)).to(dev)
    out = torch.empty((T, D), dtype=torch.float32, device=dev)
    ws = torch.empty(qt.qt_moe_layer_workspace_bytes(T, k, E, D, F), dtype=torch.uint8, device=dev)
    _, topk = workloads.moe_tokens()
    hit = len(np.unique(topk))
    for name, (gb, ub, db) in (("moe_layer", (3, 3, 3)), ("moe_layer_int4_up3", (4, 3, 4))):
        g, u, d = store["gate", gb], store["up", ub], store["down", db]

        def step(i):
            qt.qt_moe_layer(Xd, Ld, k, g, u, d, out=out, workspace=ws)

        for i in range(3):
            step(i)
        ms = time_launches(step, 20, torch)
        per_exp = sum(a[0].shape[1] + a[1][0].numel() * 4 for a in (g, u, d))
        mb = hit * per_exp + Xm.nbytes + T * D * 4
        legs[name] = {"ms": round(ms, 4), "experts_hit": hit, "bits": [gb, ub, db],
                      "GB_s": round(mb / (ms * 1e-3) / 1e9, 1), "bound": "hbm",
                      "frac": round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "bytes_per_step": int(mb), "launches": 2}
        log(f"leg {name}: {legs[name]}")
    del store, out, ws


F32_MFMA_PEAK_TFLOPS = 157.3   # dense f32 matrix cores
F64_PEAK_TFLOPS = 78.6         # f64 vector (the matrix rate is the same)


def gptq_leg(torch, qt, workloads, dev, legs):
    # ------------------------------------- GPTQ at the search shape (bf16 X)
    log("leg gptq: X[8192x17408] bf16, W[5120x17408]")
    Xb = workloads.bf16_bits_rne(workloads.search_x())
    Xd = torch.from_numpy(Xb.view(np.int16)).view(torch.bfloat16).to(dev)
    del Xb
    T, I = Xd.shape
    H = torch.empty((I, I), dtype=torch.float32, device=dev)
    ws = torch.empty(qt.qt_hessian_full_workspace_bytes(T, I, qt.QT_BF16), dtype=torch.uint8,
                     device=dev)
    qt.qt_hessian_full(Xd, H, workspace=ws)
    ms_h = time_launches(lambda i: qt.qt_hessian_full(Xd, H, workspace=ws), 3, torch)
    del ws, Xd
    fl_h = T * I * (I + 1)  # the symmetric product: T I (I + 1) / 2 multiply-adds
    U = torch.empty((I, I), dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(qt.qt_gptq_factor_workspace_bytes(I), dtype=torch.uint8, device=dev)
    qt.qt_gptq_factor(H, 0.01, U, info, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    qt.qt_gptq_factor(H, 0.01, U, info, workspace=ws)
    torch.cuda.synchronize()
    ms_f = (time.perf_counter() - t0) * 1e3
    fl_f = 2 * I ** 3 / 3  # Cholesky n^3/3 + triangular inverse n^3/3
    del ws
    W = workloads.search_w()
    O = W.shape[0]
    Wd = torch.from_numpy(W).to(dev)
    del W
    G = qt.qt_groups(I)
    s = torch.empty((O, G), dtype=torch.float32, device=dev)
    c = torch.empty((O, I), dtype=torch.int8, device=dev)
    ws = torch.empty(qt.qt_gptq_workspace_bytes(O, I), dtype=torch.uint8, device=dev)
    qt.qt_gptq_i3(Wd, U, s, c, workspace=ws)
    ms_s = time_launches(lambda i: qt.qt_gptq_i3(Wd, U, s, c, workspace=ws), 2, torch, warmup=0)
    fl_s = O * I * I  # block propagation: sum over blocks of 2 O 128 (I - b1)
    del ws
    p = qt.qt_pack_i3(c)
    ws = torch.empty(qt.qt_gptq_proxy_workspace_bytes(O, I), dtype=torch.uint8, device=dev)
    terms = qt.qt_gptq_proxy(Wd, p, s, H, workspace=ws)
    ms_p = time_launches(lambda i: qt.qt_gptq_proxy(Wd, p, s, H, terms, workspace=ws), 2, torch,
                         warmup=0)
    fl_p = 2 * 2 * O * I * I
    s0, c0, _ = qt.qt_quantize_g64(Wd, want_grid_idx=False)
    t_rtn = qt.qt_gptq_proxy(Wd, qt.qt_pack_i3(c0), s0, H, workspace=ws).cpu().numpy()
    t_g = terms.cpu().numpy()
    legs["gptq"] = {
        "hessian_full": {"ms": round(ms_h, 3), "TFLOP_s": round(fl_h / ms_h / 1e9, 1),
                         "bound": "mfma", "peak": 2500.0,
                         "frac": round(fl_h / ms_h / 1e9 / 2500.0, 4)},
        "factor": {"ms": round(ms_f, 2), "TFLOP_s": round(fl_f / ms_f / 1e9, 2), "bound": "f64",
                   "peak": F64_PEAK_TFLOPS, "frac": round(fl_f / ms_f / 1e9 / F64_PEAK_TFLOPS, 4),
                   "info": int(info.item())},
        "sweep": {"ms": round(ms_s, 3), "TFLOP_s": round(fl_s / ms_s / 1e9, 1), "bound": "mfma",
                  "peak": F32_MFMA_PEAK_TFLOPS,
                  "frac": round(fl_s / ms_s / 1e9 / F32_MFMA_PEAK_TFLOPS, 4)},
        "proxy": {"ms": round(ms_p, 3), "TFLOP_s": round(fl_p / ms_p / 1e9, 1), "bound": "mfma",
                  "peak": F32_MFMA_PEAK_TFLOPS,
                  "frac": round(fl_p / ms_p / 1e9 / F32_MFMA_PEAK_TFLOPS, 4)},
        "proxy_error": round(float(t_g[0] / t_g[1]), 6),
        "proxy_error_rtn": round(float(t_rtn[0] / t_rtn[1]), 6),
        "shape": {"T": T, "O": O, "I": I}}
    log(f"leg gptq: {legs['gptq']}")
    del H, U, Wd, s, c, p, ws, terms, s0, c0


def int4_leg(torch, qt, workloads, dev, legs, args):
    # --------------------------------------------- grouped int4, decode shape
    W, x = workloads.decode()
    O, I = W.shape
    G = qt.qt_groups(I)
    Wd = torch.from_numpy(W).to(dev)
    xd = torch.from_numpy(x).to(dev)
    s, c, _ = qt.qt_quantize_g64_i4(Wd, want_grid_idx=False)
    p = qt.qt_pack_i4(c)
    torch.cuda.synchronize()
    ms_q = time_launches(lambda i: qt.qt_quantize_g64_i4(Wd, scales=s, codes=c,
                                                         want_grid_idx=False), 20, torch)
    ms_p = time_launches(lambda i: qt.qt_pack_i4(c, p), 50, torch)
    packs = torch.empty((N_COPIES, p.numel()), dtype=torch.uint8, device=dev)
    scs = torch.empty((N_COPIES, O, G), dtype=torch.float32, device=dev)
    packs.copy_(p.expand(N_COPIES, -1))
    scs.copy_(s.expand(N_COPIES, -1, -1))
    y = torch.empty(O, dtype=torch.float32, device=dev)
    bytes_step = p.numel() + s.numel() * 4 + I * 4 + O * 4
    ms, _ = graph_ms(lambda j: qt.qt_matvec_i4(packs[j], scs[j], O, I, xd, y), N_COPIES,
                     args.warmup, args.steps, torch)
    gbs = bytes_step / (ms * 1e-3) / 1e9
    legs["gemv_decode_int4"] = {"us": round(ms * 1e3, 3), "GB_s": round(gbs, 1), "bound": "hbm",
                                "frac": round(gbs / HBM_PEAK_GBS, 4),
                                "bytes_per_launch": int(bytes_step),
                                "kernel": "gemv_batch_kernel<128,16,1,128,f32,vec,int4>"}
    legs["quantize_rtn_decode_int4"] = {"ms": round(ms_q, 5),
                                        "groups_per_s": round(O * G / (ms_q * 1e-3))}
    bytes_p = O * I + p.numel()
    legs["pack_decode_int4"] = {"ms": round(ms_p, 5),
                                "GB_s": round(bytes_p / (ms_p * 1e-3) / 1e9, 1)}
    log(f"leg int4: {legs['gemv_decode_int4']} {legs['quantize_rtn_decode_int4']} "
        f"{legs['pack_decode_int4']}")
    del packs, scs


def quant_leg(torch, qt, workloads, dev, legs):
    # -------------------------------------------------------- quantize + pack (decode, RTN)
    W, _ = workloads.decode()
    O, I = W.shape
    G = qt.qt_groups(I)
    Wd = torch.from_numpy(W).to(dev)
    s = torch.empty((O, G), dtype=torch.float32, device=dev)
    c = torch.empty((O, I), dtype=torch.int8, device=dev)
    p = torch.empty(qt.qt_packed_bytes(O, I), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: qt.qt_quantize_g64(Wd, None, 0, scales=s, codes=c,
                                                   want_grid_idx=False), 50, torch)
    bytes_q = O * I * 4 + O * I + O * G * 4
    legs["quantize_rtn_decode"] = {"ms": round(ms, 5), "groups_per_s": round(O * G / (ms * 1e-3)),
                                   "GB_s": round(bytes_q / (ms * 1e-3) / 1e9, 1),
                                   "bound": "hbm", "frac": round(bytes_q / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    ms = time_launches(lambda i: qt.qt_pack_i3(c, p), 50, torch)
    bytes_p = O * I + p.numel()
    legs["pack_decode"] = {"ms": round(ms, 5), "GB_s": round(bytes_p / (ms * 1e-3) / 1e9, 1),
                           "bound": "hbm", "frac": round(bytes_p / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"leg quantize/pack decode: {legs['quantize_rtn_decode']} {legs['pack_decode']}")
    del Wd, s, c, p


def search_leg(torch, qt, workloads, dev, legs):
    # -------------------------------------------------------- Hessian diagonal + search
    log("leg search: generating X[8192x17408], W[5120x17408]")
    X = workloads.search_x()
    Xd = torch.from_numpy(X).to(dev)
    del X
    T, I = Xd.shape
    d = torch.empty(I, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, qt.qt_hessian_workspace_bytes(T, I)), dtype=torch.uint8, device=dev)
    ms = time_launches(lambda i: qt.qt_hessian_diag(Xd, d, workspace=ws), 20, torch)
    hb = T * I * 4 + I * 4
    legs["hessian_diag"] = {"ms": round(ms, 5), "GB_s": round(hb / (ms * 1e-3) / 1e9, 1),
                            "bound": "hbm", "frac": round(hb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"leg hessian: {legs['hessian_diag']}")
    del Xd, ws
    W = workloads.search_w()
    O, I = W.shape
    G = qt.qt_groups(I)
    Wd = torch.from_numpy(W).to(dev)
    del W
    s = torch.empty((O, G), dtype=torch.float32, device=dev)
    c = torch.empty((O, I), dtype=torch.int8, device=dev)
    k = torch.empty((O, G), dtype=torch.uint8, device=dev)
    qt.qt_quantize_g64(Wd, d, 64, 0.5, 1.0, scales=s, codes=c, grid_idx=k)
    ms = time_launches(lambda i: qt.qt_quantize_g64(Wd, d, 64, 0.5, 1.0, scales=s, codes=c,
                                                   grid_idx=k), 3, torch)
    ngroups = O * G
    # per group: 64 candidates x 64 slots x 9 operations (divide, round, max,
    # min, multiply, subtract, multiply, multiply, add)
    ops = ngroups * 64 * 64 * 9
    legs["quantize_search"] = {"ms": round(ms, 4), "groups_per_s": round(ngroups / (ms * 1e-3)),
                               "bound": "alu", "achieved_Tops": round(ops / (ms * 1e-3) / 1e12, 2),
                               "peak_Tops": round(VALU_PEAK_TOPS, 2),
                               "frac": round(ops / (ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                               "op_count": "9 per slot per candidate (division as one)"}
    log(f"leg search: {legs['quantize_search']}")
    # two-stage signed search: 2 x 64 signed candidates, then 32 refinement points
    qt.qt_quantize_g64_signed(Wd, d, 64, 32, 0.5, 1.0, scales=s, codes=c)
    ms = time_launches(lambda i: qt.qt_quantize_g64_signed(Wd, d, 64, 32, 0.5, 1.0, scales=s,
                                                          codes=c), 3, torch)
    ops = ngroups * (2 * 64 + 32) * 64 * 9
    legs["quantize_search_signed"] = {"ms": round(ms, 4), "groups_per_s": round(ngroups / (ms * 1e-3)),
                                      "bound": "alu", "achieved_Tops": round(ops / (ms * 1e-3) / 1e12, 2),
                                      "peak_Tops": round(VALU_PEAK_TOPS, 2),
                                      "frac": round(ops / (ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                                      "candidates": "2 x 64 + 32 per group"}
    log(f"leg search signed: {legs['quantize_search_signed']}")
    del Wd, s, c, k, d


def moe_leg(torch, qt, workloads, dev, legs, int3_step=True, int4_steps=False):
    # -------------------------------------------------------- grouped MoE GEMV
    E = workloads.MOE_EXPERTS
    log("leg moe: generating and quantizing 128 experts x (up, down)")
    shapes = {"up": workloads.MOE_UP_SHAPE, "down": workloads.MOE_DOWN_SHAPE}
    need = set()
    if int3_step:
        need |= {("up", 3), ("down", 3)}
    if int4_steps:
        need |= {("up", 4), ("down", 4), ("up", 3)}
    fmt = {3: (qt.qt_packed_bytes, qt.qt_quantize_g64, qt.qt_pack_i3),
           4: (qt.qt_packed_bytes_i4, qt.qt_quantize_g64_i4, qt.qt_pack_i4)}
    store = {}
    for proj, bits in need:
        O_, I_ = shapes[proj]
        store[proj, bits] = (
            torch.empty((E, fmt[bits][0](O_, I_)), dtype=torch.uint8, device=dev),
            torch.empty((E, O_, qt.qt_groups(I_)), dtype=torch.float32, device=dev))
    for proj in ("up", "down"):
        bl = sorted(b for (pr, b) in need if pr == proj)
        for e0 in range(0, E, 16):
            mats = workloads.moe_experts_parallel(proj, range(e0, e0 + 16), workers=16)
            for j, m in enumerate(mats):
                md = torch.from_numpy(m).to(dev)
                for bits in bl:
                    pk, sc = store[proj, bits]
                    s_, c_, _ = fmt[bits][1](md, want_grid_idx=False)
                    sc[e0 + j].copy_(s_)
                    fmt[bits][2](c_, pk[e0 + j])
            torch.cuda.synchronize()
    (Ou, Iu), (Od, Id) = shapes["up"], shapes["down"]
    Xm, top = workloads.moe_tokens()
    tok, exp, offs = workloads.route_pairs(top, E)
    P = tok.size
    Xmd = torch.from_numpy(Xm).to(dev)
    tokd = torch.from_numpy(tok).to(dev)
    offd = torch.from_numpy(offs).to(dev)
    h = torch.empty((P, Ou), dtype=torch.float32, device=dev)
    yo = torch.empty((P, Od), dtype=torch.float32, device=dev)
    hit = int(np.count_nonzero(np.diff(offs)))
    grouped = {3: qt.qt_matvec_i3_grouped, 4: qt.qt_matvec_i4_grouped}

    steps = []
    if int3_step:
        steps.append(("moe_grouped", 3, 3))
    if int4_steps:
        steps += [("moe_grouped_int4", 4, 4), ("moe_grouped_int4_up3", 3, 4)]
    for name, bu, bd in steps:
        pu, su = store["up", bu]
        pdn, sdn = store["down", bd]

        def moe_step(i):
            grouped[bu](pu, su, E, Ou, Iu, Xmd, offd, P, pair_row=tokd, Y=h)
            grouped[bd](pdn, sdn, E, Od, Id, h, offd, P, Y=yo)

        for i in range(5):
            moe_step(i)
        ms = time_launches(moe_step, 20, torch)
        per_exp = pu.shape[1] + su[0].numel() * 4 + pdn.shape[1] + sdn[0].numel() * 4
        mb = hit * per_exp + Xm.nbytes + P * (Ou + Od) * 4 * 2
        legs[name] = {"ms": round(ms, 4), "experts_hit": hit, "pairs": int(P),
                      "up_bits": bu, "down_bits": bd,
                      "GB_s": round(mb / (ms * 1e-3) / 1e9, 1), "bound": "hbm",
                      "frac": round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "bytes_per_step": int(mb)}
        log(f"leg {name}: {legs[name]}")
    del store, h, yo


def prefill_leg(torch, qt, workloads, dev, legs):
    # -------------------------------------------------------- prefill GEMM (bf16 MFMA)
    log("leg prefill: generating and quantizing W[18432x7168]")
    O, I = workloads.PREFILL_SHAPE
    G = qt.qt_groups(I)
    pp = torch.empty(qt.qt_packed_bytes(O, I), dtype=torch.uint8, device=dev)
    sp = torch.empty((O, G), dtype=torch.float32, device=dev)
    for slab in range(O // 1024):
        m = torch.from_numpy(workloads.prefill_w([slab])).to(dev)
        s_, c_, _ = qt.qt_quantize_g64(m, want_grid_idx=False)
        sp[slab * 1024:(slab + 1) * 1024].copy_(s_)
        qt.qt_pack_i3(c_, pp[slab * 1024 * G * 24:(slab + 1) * 1024 * G * 24])
    Xb = workloads.prefill_x()
    Xbd = torch.from_numpy(Xb.view(np.int16)).view(torch.bfloat16).to(dev)
    B = Xbd.shape[0]
    Y = torch.empty((B, O), dtype=torch.float32, device=dev)
    for i in range(3):
        qt.qt_matmul_i3(pp, sp, O, I, Xbd, Y)
    ms = time_launches(lambda i: qt.qt_matmul_i3(pp, sp, O, I, Xbd, Y), 20, torch)
    flops = 2.0 * B * O * I
    tf = flops / (ms * 1e-3) / 1e12
    legs["prefill_gemm"] = {"ms": round(ms, 4), "TFLOP_s": round(tf, 1), "bound": "mfma",
                            "peak_TFLOP_s": BF16_PEAK_TFLOPS, "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    log(f"leg prefill: {legs['prefill_gemm']}")


def cpu_baseline(W, x, seconds, bytes_step):
    """The CPU oracle's fp64 dequantize-then-multiply of the same decode
    matrix, repeated for about `seconds` on one host core."""
    import oracle

    O, I = W.shape
    s, c, _ = oracle.quantize_g64(W)
    p = oracle.pack_i3(c)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        oracle.matvec_f64(p, s, O, I, x)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(bytes_step * n / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} fp64 dequantize-then-multiply passes over the decode matrix "
                      f"W[{O}x{I}] ({dt:.1f} s, single thread)"}


if __name__ == "__main__":
    main()
