"""Benchmark of the int3-g64 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs all|gemv|LEG[,LEG...]]

Headline (one JSON line on stdout): the decode GEMV, W[2048x7168] int3-g64
with f32 scales times x[7168] f32, batch 1.  A step is one dequantize-multiply
of the whole matrix; consecutive steps read 64 distinct copies of the packed
weights (64 x 6.46 MB = 413 MB, more than the 256 MB Infinity Cache), so every
step streams its weights from HBM.  The 64 launches are captured in one HIP
graph; each replay is timed by its own pair of events on the stream the
kernels run on, and the reported time per launch is the median over the
replays (p10 and p90 beside it).  value = algorithmic bytes per step (packed
weights + scales + x + y = 6,459,392 B) / median time per launch.

Beside the headline: the same multiply on the tail variant W[2048x7200] (113
groups, the last one 32 wide), the same kernel over all 64 copies as one
matrix in a single launch (O = 131072, 413 MB: the streaming rate without
launch gaps), and a measured streaming-read peak (a device reduction over
1 GiB) that the GEMV rates are also quoted against.

The other rows of the hot path are timed as "legs" on their own workloads:
the Hessian diagonal and the weighted scale search (W[5120x17408],
X[8192x17408]), plain quantize + pack at the decode shape, the grouped MoE
GEMV (128 experts, 32 tokens, top-8) and the bf16 MFMA prefill GEMM
(X[512x7168] x W[18432x7168]); grouped int4: the decode GEMV with int4
weights and the MoE step with every projection at int4 and with up at int3
(the per-projection mix); GPTQ and the MoE expert layer.  Every input is
seeded synthetic data (workloads.py) resident on the GPU before its timed
region starts.  The CPU oracle is timed beside the legs on bounded samples
(bench_cpu.py), on one host thread and on N threads.
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
# Vector ALU issue peak: 128 lanes per clock per CU at 2.4 GHz = 78.64 T
# lane-instructions/s (the published 157.3 TFLOP/s fp32 vector peak with an
# FMA as two flops).  The search legs' roofline fraction is the kernel's
# executed vector instructions (SQ_INSTS_VALU of a counter pass, times 64
# lanes) per second of its live time against this peak.
VALU_ISSUE_PEAK = 256 * 128 * 2.4e9
N_COPIES = 64
MIN_REPLAYS = 8  # timed graph replays of the headline (>= 512 launches)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--legs", default="all",
                    help="all, gemv (headline only) or a comma list of: " + ",".join(LEG_NAMES))
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="CPU-oracle time per baseline measurement (1 thread and N threads each)")
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


def counters_for(name):
    """Counter figures of a kernel from profiles/<name>_counters.json, if the
    kernel source is unchanged since they were taken; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha") != sha_of(*rec.get("sources", [])):
        return None
    return rec


def valu_roofline(cnt, ms):
    """ALU roofline of a kernel from its executed vector instructions (a
    counter record of the same kernel source) and its live time in ms."""
    if cnt is None:
        return {"bound": "alu", "achieved": None, "peak": VALU_ISSUE_PEAK / 1e12,
                "unit": "T lane-instructions/s", "frac": None}
    rate = cnt["valu_wave_insts"] * 64 / (ms * 1e-3)
    return {"bound": "alu", "achieved": round(rate / 1e12, 2), "peak": round(VALU_ISSUE_PEAK / 1e12, 2),
            "unit": "T lane-instructions/s", "frac": round(rate / VALU_ISSUE_PEAK, 4),
            "valu_wave_insts": cnt["valu_wave_insts"]}


MOE_ROUNDS, MOE_CALLS = 9, 4  # interleaved timing rounds of the MoE steps
PREFILL_COPIES = 6  # weight copies the prefill GEMM's rotating figure cycles through
SETTLE_S = 1.0  # untimed sustained run before a leg is timed


def settle(fns, torch, seconds=SETTLE_S):
    """Run the leg's own work (each fn in turn) for about `seconds`, untimed:
    a sustained load runs at a drifting rate for its first second or so (the
    clock and power settling after the host-side set-up of the leg), so the
    timed rounds start from the steady state."""
    t_end = time.perf_counter() + seconds
    i = 0
    while True:
        for fn in fns:
            fn(i)
        i += 1
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break


def time_launches(fn, n, torch, warmup=2, settle_s=0.0):
    """Average time per fn() call over n back-to-back calls, from a pair of
    events on the current stream (the stream the kernels run on), after
    `warmup` untimed calls (and, with settle_s, a sustained untimed run)."""
    if settle_s > 0:
        settle([fn], torch, settle_s)
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
    """Median per-call time of fn(j), j = 0..n_copies-1, captured once in a
    HIP graph and replayed (so that host-side call overhead does not pace the
    GPU); -> (ms per call, calls timed)."""
    reps = max(MIN_REPLAYS, -(-steps // n_copies))
    return graph_replays(fn, n_copies, warmup, reps, torch)["median"], reps * n_copies


def graph_replays(fn, n_copies, warmup, reps, torch):
    """Capture fn(0..n_copies-1) in one HIP graph on a side stream and time
    `reps` replays, each between its own pair of events recorded on that
    stream; -> {"median", "p10", "p90"} of the per-call time in ms."""
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        for j in range(n_copies):
            fn(j)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for j in range(n_copies):
            fn(j)
    with torch.cuda.stream(cs):
        for _ in range(max(1, -(-warmup // n_copies))):
            graph.replay()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(cs)
        for r in range(reps):
            graph.replay()
            evs[r + 1].record(cs)
        torch.cuda.synchronize()
    per = np.array([evs[r].elapsed_time(evs[r + 1]) for r in range(reps)]) / n_copies
    return {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
            "p90": float(np.percentile(per, 90))}


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

    reps = max(MIN_REPLAYS, -(-args.steps // N_COPIES))
    log(f"decode GEMV: graph of {N_COPIES} launches, {reps} timed replays")
    tm = graph_replays(gemv, N_COPIES, args.warmup, reps, torch)
    steps = reps * N_COPIES
    ms_step = tm["median"]
    value = bytes_step / (ms_step * 1e-3) / 1e9
    tr = traffic_for("gemv_decode", bytes_step)
    roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                "traffic": tr, "kernel": "gemv_decode1_kernel<3>",
                "launch_us_median": round(ms_step * 1e3, 3),
                "launch_us_p10": round(tm["p10"] * 1e3, 3),
                "launch_us_p90": round(tm["p90"] * 1e3, 3),
                "bytes_per_launch": bytes_step}
    log(f"  {ms_step * 1e3:.3f} us/launch median (p10 {tm['p10'] * 1e3:.3f}, p90 "
        f"{tm['p90'] * 1e3:.3f}) = {value:.0f} GB/s")

    # the same kernel over the 64 copies as one matrix, one launch
    Ostack = O * N_COPIES
    ystack = torch.empty(Ostack, dtype=torch.float32, device=dev)
    stack_bytes = packs.numel() + scs.numel() * 4 + I * 4 + Ostack * 4
    # untimed warm-up: the first second or so of a sustained stream like this
    # one runs at a drifting rate (113-140 us per launch, then a steady
    # 106-109 us on the same data), while short launches like the decode
    # graph's hold their rate from the start
    settle([lambda i: qt.qt_matvec_i3(packs.view(-1), scs.view(-1), Ostack, I, xd, ystack)],
           torch, 1.5)
    # seven rounds of five launches, the median round
    rounds = [time_launches(lambda i: qt.qt_matvec_i3(packs.view(-1), scs.view(-1), Ostack, I,
                                                      xd, ystack), 5, torch, warmup=1)
              for _ in range(7)]
    ms = float(np.median(rounds))
    gbs = stack_bytes / (ms * 1e-3) / 1e9
    legs["gemv_stacked_one_launch"] = {
        "us": round(ms * 1e3, 2),
        "us_rounds_min_max": [round(min(rounds) * 1e3, 2), round(max(rounds) * 1e3, 2)],
        "GB_s": round(gbs, 1), "bound": "hbm",
        "frac": round(gbs / HBM_PEAK_GBS, 4), "O": Ostack, "I": I,
        "bytes_per_launch": int(stack_bytes), "traffic": traffic_for("gemv_stacked", stack_bytes)}
    log(f"leg gemv_stacked_one_launch: {legs['gemv_stacked_one_launch']}")
    del packs, scs, ystack

    # tail variant: W[2048x7200], 113 groups, the last one 32 wide
    Wt, xt = workloads.decode(tail=True)
    Ot, It = Wt.shape
    Gt = qt.qt_groups(It)
    st, ct, _ = qt.qt_quantize_g64(torch.from_numpy(Wt).to(dev))
    pt = qt.qt_pack_i3(ct)
    xtd = torch.from_numpy(xt).to(dev)
    packs_t = torch.empty((N_COPIES, pt.numel()), dtype=torch.uint8, device=dev)
    scs_t = torch.empty((N_COPIES, Ot, Gt), dtype=torch.float32, device=dev)
    packs_t.copy_(pt.expand(N_COPIES, -1))
    scs_t.copy_(st.expand(N_COPIES, -1, -1))
    yt = torch.empty(Ot, dtype=torch.float32, device=dev)
    bytes_t = pt.numel() + st.numel() * 4 + It * 4 + Ot * 4
    tmt = graph_replays(lambda j: qt.qt_matvec_i3(packs_t[j], scs_t[j], Ot, It, xtd, yt),
                        N_COPIES, args.warmup, reps, torch)
    gbs = bytes_t / (tmt["median"] * 1e-3) / 1e9
    legs["gemv_decode_tail_7200"] = {
        "us_median": round(tmt["median"] * 1e3, 3), "us_p10": round(tmt["p10"] * 1e3, 3),
        "us_p90": round(tmt["p90"] * 1e3, 3), "GB_s": round(gbs, 1), "bound": "hbm",
        "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": int(bytes_t),
        "O": Ot, "I": It}
    log(f"leg gemv_decode_tail_7200: {legs['gemv_decode_tail_7200']}")
    del packs_t, scs_t

    # measured streaming peak: a 1 GiB device-to-device copy (bytes read plus
    # bytes written over its time) and a device sum over the same 1 GiB (bytes
    # read); the larger is the streaming peak the GEMV rates are quoted against
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    big2 = torch.empty_like(big)
    for _ in range(3):
        big2.copy_(big)
        big.sum()
    ms_c = time_launches(lambda i: big2.copy_(big), 10, torch)
    ms_s = time_launches(lambda i: big.sum(), 10, torch)
    copy_gbs = 2 * big.numel() * 4 / (ms_c * 1e-3) / 1e9
    sum_gbs = big.numel() * 4 / (ms_s * 1e-3) / 1e9
    stream_peak = max(copy_gbs, sum_gbs)
    del big, big2
    log(f"streaming peak: 1 GiB copy {copy_gbs:.0f} GB/s (read + write), sum {sum_gbs:.0f} GB/s")

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

    cpu = cpu_baselines(args.cpu_seconds, legs, W, x)

    line = {
        "metric": "int3-g64 GEMV effective HBM GB/s (% of peak) at I=7168; quantize groups/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "pct_of_stream_peak": round(100 * value / stream_peak, 2),
        "stream_peak_GB_s": round(stream_peak, 1),
        "stream_probe_GB_s": {"copy_1GiB_read_plus_write": round(copy_gbs, 1),
                              "sum_1GiB_read": round(sum_gbs, 1)},
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
        "timing": {"replays": reps, "launches_per_replay": N_COPIES,
                   "per_launch_ms_median": round(ms_step, 6),
                   "per_launch_ms_p10": round(tm["p10"], 6),
                   "per_launch_ms_p90": round(tm["p90"], 6)},
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
    schemes = (("moe_layer", (3, 3, 3)), ("moe_layer_int4_up3", (4, 3, 4)))

    def make_step(gb, ub, db):
        g, u, d = store["gate", gb], store["up", ub], store["down", db]

        def step(i):
            qt.qt_moe_layer(Xd, Ld, k, g, u, d, out=out, workspace=ws)

        return step, sum(a[0].shape[1] + a[1][0].numel() * 4 for a in (g, u, d))

    fns = {name: make_step(*bits) for name, bits in schemes}
    settle([fn for fn, _ in fns.values()], torch)
    rounds = {name: [] for name in fns}  # interleaved, as the MoE steps
    for r in range(MOE_ROUNDS):
        for name, (fn, _) in fns.items():
            rounds[name].append(time_launches(fn, MOE_CALLS, torch, warmup=1))
    for name, (gb, ub, db) in schemes:
        ms = float(np.median(rounds[name]))
        mb = hit * fns[name][1] + Xm.nbytes + T * D * 4
        legs[name] = {"ms": round(ms, 4), "ms_rounds_min_max": [round(min(rounds[name]), 4),
                                                                round(max(rounds[name]), 4)],
                      "experts_hit": hit, "bits": [gb, ub, db],
                      "GB_s": round(mb / (ms * 1e-3) / 1e9, 1), "bound": "hbm",
                      "frac": round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "bytes_per_step": int(mb), "launches": 5}
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
    ms_h = time_launches(lambda i: qt.qt_hessian_full(Xd, H, workspace=ws), 3, torch,
                        settle_s=SETTLE_S)
    del ws, Xd
    fl_h = T * I * (I + 1)  # the symmetric product: T I (I + 1) / 2 multiply-adds
    U = torch.empty((I, I), dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(qt.qt_gptq_factor_workspace_bytes(I), dtype=torch.uint8, device=dev)
    settle([lambda i: qt.qt_gptq_factor(H, 0.01, U, info, workspace=ws)], torch)
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
    ms_s = time_launches(lambda i: qt.qt_gptq_i3(Wd, U, s, c, workspace=ws), 2, torch, warmup=0,
                         settle_s=SETTLE_S)
    fl_s = O * I * I  # block propagation: sum over blocks of 2 O 128 (I - b1)
    del ws
    p = qt.qt_pack_i3(c)
    ws = torch.empty(qt.qt_gptq_proxy_workspace_bytes(O, I), dtype=torch.uint8, device=dev)
    terms = qt.qt_gptq_proxy(Wd, p, s, H, workspace=ws)
    ms_p = time_launches(lambda i: qt.qt_gptq_proxy(Wd, p, s, H, terms, workspace=ws), 2, torch,
                         warmup=0, settle_s=SETTLE_S)
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
                                                         want_grid_idx=False), 20, torch,
                         settle_s=SETTLE_S)
    ms_p = time_launches(lambda i: qt.qt_pack_i4(c, p), 50, torch, settle_s=SETTLE_S)
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
                                "kernel": "gemv_decode1_kernel<4>"}
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
                                                   want_grid_idx=False), 50, torch,
                       settle_s=SETTLE_S)
    bytes_q = O * I * 4 + O * I + O * G * 4
    legs["quantize_rtn_decode"] = {"ms": round(ms, 5), "groups_per_s": round(O * G / (ms * 1e-3)),
                                   "GB_s": round(bytes_q / (ms * 1e-3) / 1e9, 1),
                                   "bound": "hbm", "frac": round(bytes_q / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    ms = time_launches(lambda i: qt.qt_pack_i3(c, p), 50, torch, settle_s=SETTLE_S)
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
    ms = time_launches(lambda i: qt.qt_hessian_diag(Xd, d, workspace=ws), 20, torch,
                       settle_s=SETTLE_S)
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
                                                   grid_idx=k), 3, torch, settle_s=SETTLE_S)
    ngroups = O * G
    # per group: 64 candidates x 64 slots x 9 operations (divide, round, max,
    # min, multiply, subtract, multiply, multiply, add)
    ops = ngroups * 64 * 64 * 9
    legs["quantize_search"] = dict(
        {"ms": round(ms, 4), "groups_per_s": round(ngroups / (ms * 1e-3)),
         "ops_Tops": round(ops / (ms * 1e-3) / 1e12, 2),
         "op_count": "9 per slot per candidate (division as one)"},
        **valu_roofline(counters_for("search"), ms))
    log(f"leg search: {legs['quantize_search']}")
    # two-stage signed search: 2 x 64 signed candidates, then 32 refinement points
    qt.qt_quantize_g64_signed(Wd, d, 64, 32, 0.5, 1.0, scales=s, codes=c)
    ms = time_launches(lambda i: qt.qt_quantize_g64_signed(Wd, d, 64, 32, 0.5, 1.0, scales=s,
                                                          codes=c), 3, torch, settle_s=SETTLE_S)
    ops = ngroups * (2 * 64 + 32) * 64 * 9
    legs["quantize_search_signed"] = dict(
        {"ms": round(ms, 4), "groups_per_s": round(ngroups / (ms * 1e-3)),
         "ops_Tops": round(ops / (ms * 1e-3) / 1e12, 2), "candidates": "2 x 64 + 32 per group"},
        **valu_roofline(counters_for("search_signed"), ms))
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
    def make_step(bu, bd):
        pu, su = store["up", bu]
        pdn, sdn = store["down", bd]

        def moe_step(i):
            grouped[bu](pu, su, E, Ou, Iu, Xmd, offd, P, pair_row=tokd, Y=h)
            grouped[bd](pdn, sdn, E, Od, Id, h, offd, P, Y=yo)

        per_exp = pu.shape[1] + su[0].numel() * 4 + pdn.shape[1] + sdn[0].numel() * 4
        return moe_step, per_exp

    fns = {name: make_step(bu, bd) for name, bu, bd in steps}
    settle([fn for fn, _ in fns.values()], torch)
    # the steps are timed in interleaved rounds (each round times every step
    # over MOE_CALLS calls), and each reports its median round: the GPU's
    # clock settles during the first hundreds of milliseconds of load, which
    # would otherwise slow whichever step is timed first
    rounds = {name: [] for name in fns}
    for r in range(MOE_ROUNDS):
        for name, (fn, _) in fns.items():
            rounds[name].append(time_launches(fn, MOE_CALLS, torch, warmup=1))
    for name, bu, bd in steps:
        ms = float(np.median(rounds[name]))
        mb = hit * fns[name][1] + Xm.nbytes + P * (Ou + Od) * 4 * 2
        legs[name] = {"ms": round(ms, 4), "ms_rounds_min_max": [round(min(rounds[name]), 4),
                                                                round(max(rounds[name]), 4)],
                      "experts_hit": hit, "pairs": int(P),
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
    ms = time_launches(lambda i: qt.qt_matmul_i3(pp, sp, O, I, Xbd, Y), 20, torch,
                       settle_s=SETTLE_S)
    # the same multiply over PREFILL_COPIES copies of the weights in turn
    # (347 MB, more than the 256 MB Infinity Cache), as consecutive layers
    # would read them: the single-copy figure above reads weights that stay
    # in that cache between launches
    packs = torch.empty((PREFILL_COPIES, pp.numel()), dtype=torch.uint8, device=dev)
    scs = torch.empty((PREFILL_COPIES, O, G), dtype=torch.float32, device=dev)
    packs.copy_(pp.expand(PREFILL_COPIES, -1))
    scs.copy_(sp.expand(PREFILL_COPIES, -1, -1))
    ms_rot = time_launches(
        lambda i: qt.qt_matmul_i3(packs[i % PREFILL_COPIES], scs[i % PREFILL_COPIES], O, I, Xbd,
                                  Y), 4 * PREFILL_COPIES, torch, settle_s=SETTLE_S)
    del packs, scs
    flops = 2.0 * B * O * I
    tf = flops / (ms * 1e-3) / 1e12
    tf_rot = flops / (ms_rot * 1e-3) / 1e12
    legs["prefill_gemm"] = {"ms": round(ms, 4), "TFLOP_s": round(tf, 1), "bound": "mfma",
                            "peak_TFLOP_s": BF16_PEAK_TFLOPS, "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                            "rotating_copies": {"copies": PREFILL_COPIES, "ms": round(ms_rot, 4),
                                                "TFLOP_s": round(tf_rot, 1),
                                                "frac": round(tf_rot / BF16_PEAK_TFLOPS, 4)}}
    log(f"leg prefill: {legs['prefill_gemm']}")


# ---------------------------------------------------------------- CPU oracle baselines
def host_threads():
    """Host threads for the CPU baselines: the cores this process may run on,
    at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(items, seconds, threads):
    """items: callables, each one oracle call returning the units of work it
    did.  Runs them round-robin for about `seconds` on `threads` host threads
    (a ctypes call releases the interpreter lock, so the C oracle runs in
    parallel) -> (units per second, calls made)."""
    from concurrent.futures import ThreadPoolExecutor
    done_units, calls = 0.0, 0
    t0 = time.perf_counter()
    if threads == 1:
        while True:
            done_units += items[calls % len(items)]()
            calls += 1
            if time.perf_counter() - t0 >= seconds:
                break
    else:
        with ThreadPoolExecutor(threads) as ex:
            while True:
                batch = [items[(calls + k) % len(items)] for k in range(threads)]
                done_units += sum(ex.map(lambda f: f(), batch))
                calls += threads
                if time.perf_counter() - t0 >= seconds:
                    break
    return done_units / (time.perf_counter() - t0), calls


def cpu_baselines(seconds, legs, Wdec, xdec):
    """The oracle (plain scalar C, built -O2 without fast-math, never tuned for
    speed) timed on bounded samples of the legs' workloads, on one host thread
    and on N; each figure is attached to its leg as "cpu_oracle" and the
    decode matvec is the line's cpu_baseline."""
    import oracle
    import workloads
    n = host_threads()
    out = {}

    def measure(name, items, unit, sample):
        r1, c1 = oracle_rate(items, seconds, 1)
        rn, cn = oracle_rate(items, seconds, n)
        out[name] = {"unit": unit, "single_thread": round(r1, 4), "threads": n,
                     "all_threads": round(rn, 4), "sample": sample}
        log(f"cpu oracle {name}: 1 thread {r1:.4g}, {n} threads {rn:.4g} {unit}")

    O, I = Wdec.shape
    G = -(-I // 64)
    rows = 128
    slabs = []
    for r0 in range(0, O, rows):
        so, co, _ = oracle.quantize_g64(Wdec[r0:r0 + rows])
        slabs.append((so, co, oracle.pack_i3(co), Wdec[r0:r0 + rows]))
    per_row = G * 28  # packed + scale bytes of a row
    measure("matvec_decode",
            [lambda sl=sl: (oracle.matvec_f64(sl[2], sl[0], rows, I, xdec),
                            rows * per_row + I * 4 + rows * 4)[1] for sl in slabs],
            "bytes_per_s", f"fp64 dequantize-then-multiply of 128-row slabs of W[{O}x{I}]")
    measure("quantize_rtn_decode",
            [lambda sl=sl: (oracle.quantize_g64(sl[3]), rows * G)[1] for sl in slabs],
            "groups_per_s", f"plain absmax/4 quantize of 128-row slabs of W[{O}x{I}]")
    measure("pack_decode",
            [lambda sl=sl: (oracle.pack_i3(sl[1]), rows * I + rows * G * 24)[1] for sl in slabs],
            "bytes_per_s", f"bit-plane pack of 128-row slabs of the codes of W[{O}x{I}]")
    # weighted search on rows of the search matrix (importance d drawn lognormal)
    Os, Is = workloads.SEARCH_SHAPE
    Gs = -(-Is // 64)
    Ws = workloads.generic_weights(32, Is, seed=31)
    d = np.exp(workloads.generic_vector(Is, seed=32)).astype(np.float32)
    measure("quantize_search",
            [lambda k=k: (oracle.quantize_g64(Ws[4 * k:4 * k + 4], d, 64, 0.5, 1.0), 4 * Gs)[1]
             for k in range(8)],
            "groups_per_s", f"64-point weighted search of 4-row slabs of [x{Is}] rows")
    measure("quantize_search_signed",
            [lambda k=k: (oracle.quantize_g64_signed(Ws[2 * k:2 * k + 2], d, 64, 32, 0.5, 1.0),
                          2 * Gs)[1] for k in range(16)],
            "groups_per_s", f"two-stage signed 64/32 search of 2-row slabs of [x{Is}] rows")
    Xh = workloads.generic_matrix(512, Is, seed=33)
    measure("hessian_diag",
            [lambda k=k: (oracle.hessian_diag(Xh[64 * k:64 * k + 64]), 64 * Is * 4)[1]
             for k in range(8)],
            "bytes_per_s", f"f64 column sums of squares over 64-token slabs of X[.x{Is}]")
    # grouped MoE: per-pair matvecs of two experts (up and down)
    mats = []
    for e in range(2):
        for which in ("up", "down"):
            m = workloads.moe_expert(e, which)
            so, co, _ = oracle.quantize_g64(m)
            mats.append((oracle.pack_i3(co), so, m.shape[0], m.shape[1]))
    xs = {k: workloads.generic_vector(k, seed=k) for k in (7168, 2048)}
    measure("moe_grouped",
            [lambda mt=mt: (oracle.matvec_f64(mt[0], mt[1], mt[2], mt[3], xs[mt[3]]),
                            mt[0].size + mt[1].size * 4)[1] for mt in mats],
            "bytes_per_s", "fp64 (token, expert) matvecs of the up and down matrices of two experts")
    # prefill: sampled outputs of one 1024-row slab
    Op, Ip = workloads.PREFILL_SHAPE
    sp, cp, _ = oracle.quantize_g64(workloads.prefill_w([0]))
    pp = oracle.pack_i3(cp)
    Xp = workloads.bf16_bits_to_f32(workloads.prefill_x()[:64])
    rng = workloads.rng_for("generic", 9100)
    samples = [(rng.integers(0, 64, size=256), rng.integers(0, 1024, size=256)) for _ in range(8)]
    measure("prefill_gemm",
            [lambda sm=sm: (oracle.matmul_f64_sampled(pp, sp, 1024, Ip, Xp, sm[0], sm[1]),
                            2.0 * Ip * sm[0].size)[1] for sm in samples],
            "flop_per_s", f"fp64 sampled outputs (256 per call) of a 1024-row slab of W[{Op}x{Ip}]")
    # attach to the legs that ran
    for leg, key in (("quantize_rtn_decode", "quantize_rtn_decode"), ("pack_decode", "pack_decode"),
                     ("quantize_search", "quantize_search"),
                     ("quantize_search_signed", "quantize_search_signed"),
                     ("hessian_diag", "hessian_diag"), ("moe_grouped", "moe_grouped"),
                     ("prefill_gemm", "prefill_gemm")):
        if leg in legs:
            legs[leg]["cpu_oracle"] = out[key]
    m = out["matvec_decode"]
    return {"value": round(m["all_threads"] / 1e9, 3), "unit": "GB/s", "cores": n,
            "kind": "oracle",
            "sample": f"fp64 dequantize-then-multiply of 128-row slabs of the decode matrix "
                      f"W[{O}x{I}] for about {seconds:.1f} s on {n} host threads",
            "single_thread_GB_s": round(m["single_thread"] / 1e9, 3),
            "cpu_model": cpu_model(), "legs": out}


if __name__ == "__main__":
    main()
