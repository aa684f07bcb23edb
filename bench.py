#!/usr/bin/env python3
"""Benchmark of the quantized-product hot path on one MI355X.

Headline (one JSON line on stdout): Q4_0 x Q8_0 decode at the FFN-gate shape,
M = 1, N = 12288, K = 4096.  One step = quantize the f32 activation to Q8_0
and the matvec over one copy of the 28.3 MB weight matrix, in one launch
(qmm_quantize_matvec_q4_0; the same step as two launches is reported beside
it).  Steps rotate over enough byte-identical weight copies (>= 512 MB) that
every step streams its weights from HBM, not from the 256 MB last-level
cache.  `value` is weight bytes per step / step time (GB/s), inputs resident
in HBM; the timed steps are replayed from a captured HIP graph (launching
kernels of a few microseconds from Python would measure the interpreter, not
the GPU).

Also in the line: the other decode workloads (the Q8_0 matrices of one
7B-style layer, Q2_K, Q4_K and Q6_K at 12288x4096), kernel time and GB/s
each; the prefill matmul (M = 2048, same weights), int8 TOP/s;
for each, the dominant kernel's roofline (achieved / MI355X peak) and the
oracle timed on the host cores over a bounded sample of the same workload.
The decode kernel is the whole step, so its roofline takes the timed region's
time per launch; every other kernel time comes from HIP events on the launch
stream around windows of back-to-back graph replays of that kernel (each
window at least half a millisecond of work), warmed up and alternated with
the kernels it is compared with.  `attainable` holds
the measured ceilings of the probe library (a streaming read in 24 launch
shapes, at the decode's 28.3 MB, at 1 GiB and at every decode weight size;
an int8 MFMA loop; an issue-rate loop of f32 FMAs and int8 MFMAs); each
roofline also gives its fraction of the matching one.

Synthetic data: seeded Gaussian weights (std 0.02) and activations (std 1,
1% outliers x20 for decode), quantized on the GPU by the library.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_0 matvec GB/s + %HBM peak (12288×4096, M=1); prefill int8 TOPS + %MFMA"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (no sparsity)

DEC = dict(M=1, N=12288, K=4096)
PRE = dict(M=2048, N=12288, K=4096)
# The host-side leg checks the benchmarked outputs against the oracle: the
# whole decode output and the first CHECK_ROWS token rows of the prefill,
# each output within TOL times the sum of the magnitudes of its terms.
CHECK_ROWS = 64
TOL = 1e-5


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=40, help="untimed decode steps")
    ap.add_argument("--prefill-steps", type=int, default=52, help="timed prefill steps (at least 52 are timed)")
    ap.add_argument("--prefill-warmup", type=int, default=30,
                    help="untimed prefill steps (~10 ms: lets the clock settle under the MFMA load)")
    ap.add_argument("--only", choices=["all", "decode", "prefill", "configs"], default="all")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of each oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-peaks", action="store_true",
                    help="leave out the attainable-peak probes (for counter runs of the product kernels)")
    ap.add_argument("--copies-mb", type=float, default=600.0, help="total size of the rotated weight copies")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run one plain 256 MiB device-to-device copy (scales HBM byte counters)")
    args = ap.parse_args()
    if args.steps < 1 or args.prefill_steps < 1:
        ap.error("--steps and --prefill-steps must be at least 1")
    return args


def committed_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` (FETCH_SIZE + WRITE_SIZE,
    each scaled by the plain-copy calibration) from the committed rocprofv3
    counter summary, or None when there is none or the kernel's sources no
    longer hash to what was profiled."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    keys = ("traffic_bytes_per_launch", "kernel_sources", "kernel_source_sha256")
    fields = {}
    for line in text.splitlines():
        k, _, v = line.partition(": ")
        if k in keys:
            fields[k] = v.strip()
    if len(fields) != len(keys):
        return None
    h = hashlib.sha256()
    try:
        for f in fields["kernel_sources"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
    except OSError:
        return None
    return int(fields["traffic_bytes_per_launch"]) if h.hexdigest() == fields["kernel_source_sha256"] else None


def capture(torch, launch, batch):
    """A HIP graph of `batch` back-to-back launches launch(0) .. launch(batch-1)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(batch):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    return g


def warm_up(torch, graphs, min_ms=25.0, max_reps=400):
    """Replay the graphs round-robin until at least min_ms of GPU time has
    passed, so that clocks have settled before anything is timed (the first
    milliseconds after a quiet period run measurably slower).  Returns the
    mean time of one replay (ms) over the warm-up's last round."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    done, reps, last = 0.0, 0, 0.0
    while done < min_ms and reps < max_reps:
        t0.record()
        for g in graphs:
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        last = t0.elapsed_time(t1)
        done += last
        reps += 1
    return last / len(graphs)


def replay_rounds(torch, graphs, rounds, per_window=1):
    """Times `rounds` windows of every graph, alternating between the graphs
    (so that all see the same clock conditions); a window is `per_window`
    back-to-back replays of one graph between two HIP events on the launch
    stream.  Returns per graph the list of window durations in ms.  The two
    markers of a window add about 5 us of queue start-up to it (measured:
    22 decode launches per window 7.59 us each, the same launches in one
    window of 18 replays 7.37 us), which windows of at least half a
    millisecond of work (time_kernels) keep under 1 %.  (Timing Python
    launches instead would measure the interpreter for kernels of a few
    microseconds.)"""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
          for _ in graphs]
    for r in range(rounds):
        for k, g in enumerate(graphs):
            a, b = ev[k][r]
            a.record()
            for _ in range(per_window):
                g.replay()
            b.record()
    torch.cuda.synchronize()
    return [[a.elapsed_time(b) for a, b in e] for e in ev]


def per_launch(times, launches):
    """mean, median, min and max per launch (ms) of windows of `launches` launches."""
    per = sorted(t / launches for t in times)
    n = len(per)
    med = per[n // 2] if n % 2 else 0.5 * (per[n // 2 - 1] + per[n // 2])
    return {"mean": sum(per) / n, "median": med, "min": per[0], "max": per[-1], "launches": n * launches}


WINDOW_MS = 0.5


def time_kernels(torch, launches, batch, count, warm_ms=25.0):
    """Per-launch timing (see per_launch) of each launch function in
    `launches`: graphs of `batch` launches, warmed up, then timed in
    alternating windows of back-to-back replays, each window at least
    WINDOW_MS of GPU work, until each has run at least `count` launches."""
    graphs = [capture(torch, f, batch) for f in launches]
    replay_ms = warm_up(torch, graphs, warm_ms)
    per_window = max(1, min(16, -(-WINDOW_MS // max(replay_ms, 1e-3))))
    per_window = int(per_window)
    rounds = max(1, -(-count // (batch * per_window)))
    return [per_launch(t, batch * per_window) for t in replay_rounds(torch, graphs, rounds, per_window)]


def us(d):
    """A per_launch record in microseconds, rounded."""
    return {k: (round(v * 1e3, 3) if k != "launches" else v) for k, v in d.items()}


def bench_decode(args, torch, q, synth):
    N, K = DEC["N"], DEC["K"]
    wbytes = N * q.row_bytes("q4_0", K)
    log(f"decode: generating weights {N}x{K} and quantizing on the GPU")
    w = torch.from_numpy(synth.weights(N, K, config=1)).cuda()
    wq0 = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q4_0(w, wq0, N, K)
    del w
    copies = max(2, int(args.copies_mb * 1e6 // wbytes) + 1)
    wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.activations(1, K, config=1, outlier_frac=0.01, outlier_factor=20.0)).cuda()
    xq = torch.empty(q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        """One decode step: quantize x and apply the weights, in one launch."""
        q.qmm_quantize_matvec_q4_0(wqs[i % copies], x, None, y, N, K)

    def step_two_launches(i):
        """The same step as a quantize launch followed by a matvec launch."""
        q.qmm_quantize_q8_0(x, xq, 1, K)
        q.qmm_matvec_q4_0(wqs[i % copies], xq, y, N, K)

    # exactly args.steps steps: whole replays of a graph of one step per
    # weight copy, then a graph of the remaining steps; warmed up first
    for i in range(args.warmup):
        step(i)
    reps, rem = divmod(args.steps, copies)
    g_full = capture(torch, step, copies)
    graphs = [g_full] + ([capture(torch, step, rem)] if rem else [])
    warm_up(torch, graphs)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g_full.replay()
    if rem:
        graphs[1].replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    nsteps = args.steps
    # the step launched eagerly from Python, for reference
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step_eager = t0.elapsed_time(t1) / args.steps
    # the dominant kernel is the fused kernel, the whole step: its duration
    # for the roofline is the timed region's per launch.  Beside it, timed in
    # alternating windows: the same kernel, the plain matvec and the step as
    # two launches, at least 200 launches each
    count = max(200, args.steps)
    fz, mv, two = time_kernels(torch, [step, lambda i: q.qmm_matvec_q4_0(wqs[i % copies], xq, y, N, K),
                                       step_two_launches], copies, count)
    # the output of one more step, for the check against the oracle in the
    # host-side leg (every weight copy holds the same bytes)
    step(0)
    torch.cuda.synchronize()
    y_check = y.cpu().numpy().copy()
    log(f"decode: {ms_step * 1e3:.2f} us/step over {nsteps} steps in graph replay ({ms_step_eager * 1e3:.2f} eager); "
        f"fused kernel mean {fz['mean'] * 1e3:.2f} us (median {fz['median'] * 1e3:.2f}, {fz['launches']} launches), "
        f"matvec alone {mv['mean'] * 1e3:.2f} us, two launches {two['mean'] * 1e3:.2f} us, {copies} weight copies")
    gbs_step = wbytes / (ms_step * 1e-3) / 1e9
    alg = wbytes + 4 * K + 4 * N
    gbs_kernel = alg / (ms_step * 1e-3) / 1e9
    return dict(ms_step=ms_step, ms_step_eager=ms_step_eager, ms_two=two["mean"], nsteps=nsteps, gbs=gbs_step,
                wbytes=wbytes, copies=copies, y_check=y_check,
                roofline={"kernel": "qmm::k_matvec<Q4_0, fused quantize>", "bound": "hbm",
                          "achieved": round(gbs_kernel, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs_kernel / HBM_PEAK_GBS, 4),
                          "traffic": committed_traffic("k_matvec_q4_0_fused", "12288x4096"),
                          "kernel_us_mean": round(ms_step * 1e3, 3),
                          "kernel_us_basis": f"the timed region: {nsteps} back-to-back launches of this kernel "
                                             "between two HIP events",
                          "kernel_us_windows": us(fz),
                          "algorithmic_bytes": alg,
                          "matvec_only": {"kernel": "qmm::k_matvec<Q4_0>", "us_mean": round(mv["mean"] * 1e3, 3),
                                          "us": us(mv),
                                          "achieved": round(wbytes / (mv["mean"] * 1e-3) / 1e9, 1),
                                          "traffic": committed_traffic("k_matvec_q4_0", "12288x4096")}})


def bench_small(args, torch, q, synth):
    """Latency of the 512 x 1024 Q4_0 decode (its 295 KB of weight blocks stay
    in L2, so this is a latency figure, not an HBM one) and the activation
    quantizers on their own (GB/s of f32 input)."""
    N, K = 512, 1024
    w = torch.from_numpy(synth.weights(N, K, config=0)).cuda()
    wq = torch.empty(N * q.row_bytes("q4_0", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q4_0(w, wq, N, K)
    x = torch.from_numpy(synth.activations(1, K, config=0)).cuda()
    xq = torch.empty(q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q8_0(x, xq, 1, K)
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    count = max(200, args.steps)
    fz, mv = time_kernels(torch, [lambda i: q.qmm_quantize_matvec_q4_0(wq, x, None, y, N, K),
                                  lambda i: q.qmm_matvec_q4_0(wq, xq, y, N, K)], 50, count)
    wb = N * q.row_bytes("q4_0", K)
    res = {"workload": "q4_0_matvec_512x1024", "weight_bytes": wb, "l2_resident": True,
           "fused_us": us(fz), "matvec_us": us(mv),
           "matvec_gbs": round(wb / (mv["mean"] * 1e-3) / 1e9, 1),
           "hbm_frac_flagged_l2_resident": round(wb / (mv["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"small decode 512x1024: fused {fz['mean'] * 1e3:.2f} us, matvec {mv['mean'] * 1e3:.2f} us (L2-resident)")
    quant = []
    for M, Kq in ((2048, 4096), (1, 4096)):
        X = torch.from_numpy(synth.activations(M, Kq, config=4)).cuda()
        X8 = torch.empty(M * q.row_bytes("q8_0", Kq), dtype=torch.uint8, device="cuda")
        XK = torch.empty(M * q.row_bytes("q8_k", Kq), dtype=torch.uint8, device="cuda")
        t8, tk = time_kernels(torch, [lambda i: q.qmm_quantize_q8_0(X, X8, M, Kq),
                                      lambda i: q.qmm_quantize_q8_k(X, XK, M, Kq)], 20, max(100, args.steps))
        for name, t, ob in (("q8_0", t8, X8.numel()), ("q8_k", tk, XK.numel())):
            quant.append({"quantizer": name, "M": M, "K": Kq, "in_bytes": 4 * M * Kq, "out_bytes": ob,
                          "us": us(t), "in_gbs": round(4 * M * Kq / (t["mean"] * 1e-3) / 1e9, 1),
                          "hbm_frac": round((4 * M * Kq + ob) / (t["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"quantize {name} {M}x{Kq}: {t['mean'] * 1e3:.2f} us, {quant[-1]['in_gbs']} GB/s of f32 in")
    res["quantizers"] = quant
    return res


def bench_prefill(args, torch, q, synth):
    M, N, K = PRE["M"], PRE["N"], PRE["K"]
    wbytes = N * q.row_bytes("q4_0", K)
    log(f"prefill: generating {N}x{K} weights and {M}x{K} activations")
    w = torch.from_numpy(synth.weights(N, K, config=1)).cuda()
    wq = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q4_0(w, wq, N, K)
    del w
    X = torch.from_numpy(synth.activations(M, K, config=4)).cuda()
    Xq = torch.empty(M * q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        q.qmm_quantize_q8_0(X, Xq, M, K)
        q.qmm_matmul_q4_0(wq, Xq, Y, M, N, K)

    def kernel(i):
        q.qmm_matmul_q4_0(wq, Xq, Y, M, N, K)

    # the step (quantize + matmul) and the matmul alone: graphs of 4 of each,
    # warmed up together, then replayed alternately in the same rounds so
    # both see the same clock conditions; at least 52 launches each
    for _ in range(args.prefill_warmup):
        step(0)
    B = 4
    g_step, g_kern = capture(torch, step, B), capture(torch, kernel, B)
    warm_up(torch, [g_step, g_kern])
    rounds = max(1, -(-max(args.prefill_steps, 52) // B))
    t_step, t_kern = replay_rounds(torch, [g_step, g_kern], rounds)
    st, mm = per_launch(t_step, B), per_launch(t_kern, B)
    ms_step, nsteps = st["mean"], st["launches"]
    ops = 2.0 * M * N * K
    log(f"prefill: {ms_step * 1e3:.1f} us/step (median {st['median'] * 1e3:.1f}), matmul mean {mm['mean'] * 1e3:.1f} "
        f"us (median {mm['median'] * 1e3:.1f}, {mm['min'] * 1e3:.1f}..{mm['max'] * 1e3:.1f}), {rounds} rounds of {B}")
    if ms_step < mm["mean"]:
        log("prefill: WARNING the step measured shorter than the kernel it contains")
    tops_kernel = ops / (mm["mean"] * 1e-3) / 1e12
    # the first rows of one more step, for the check against the oracle in
    # the host-side leg
    step(0)
    torch.cuda.synchronize()
    y_check = Y[:CHECK_ROWS].cpu().numpy().copy()

    def time_one(launch):
        for _ in range(4):
            launch(0)
        return time_kernels(torch, [launch], B, max(args.prefill_steps, 52))[0]

    # the same prefill with Q8_0 weights (same activations, weights from the same stream)
    w = torch.from_numpy(synth.weights(N, K, config=1)).cuda()
    wq8 = torch.empty(N * q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q8_0(w, wq8, N, K)
    del w
    t8 = time_one(lambda i: q.qmm_matmul_q8_0(wq8, Xq, Y, M, N, K))
    m8_ms = t8["mean"]
    log(f"prefill q8_0 weights: matmul {m8_ms * 1e3:.1f} us (median {t8['median'] * 1e3:.1f})")
    del wq8
    # Q5_0 weights (weights of the Q5_0 workload, the same Q8_0 activations)
    w = torch.from_numpy(synth.weights(N, K, config=10)).cuda()
    wq5 = torch.empty(N * q.row_bytes("q5_0", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q5_0(w, wq5, N, K)
    del w
    t5 = time_one(lambda i: q.qmm_matmul_q5_0(wq5, Xq, Y, M, N, K))
    m5_ms = t5["mean"]
    log(f"prefill q5_0 weights: matmul {m5_ms * 1e3:.1f} us (median {t5['median'] * 1e3:.1f})")
    del wq5
    # Q4_1 and Q5_1 weights (weights of their decode workloads, the same Q8_0 activations)
    off = {}
    for fmt, cfg in (("q4_1", 9), ("q5_1", 11)):
        w = torch.from_numpy(synth.weights(N, K, config=cfg)).cuda()
        wqf = torch.empty(N * q.row_bytes(fmt, K), dtype=torch.uint8, device="cuda")
        q.QUANTIZE_W[fmt](w, wqf, N, K)
        del w
        tf = time_one(lambda i: q.MATMUL[fmt](wqf, Xq, Y, M, N, K))
        f_ms = tf["mean"]
        log(f"prefill {fmt} weights: matmul {f_ms * 1e3:.1f} us (median {tf['median'] * 1e3:.1f})")
        off[fmt] = {"kernel": f"qmm::k_matmul_{fmt}", "kernel_us_mean": round(f_ms * 1e3, 2), "kernel_us": us(tf),
                    "achieved": round(ops / (f_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                    "frac": round(ops / (f_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                    "traffic": committed_traffic(f"k_matmul_{fmt}", "2048x12288x4096")}
        del wqf
    # Q2_K weights x Q8_K activations (same shape, inputs of the Q2_K workload)
    w = torch.from_numpy(synth.weights(N, K, config=3)).cuda()
    wq2 = torch.empty(N * q.row_bytes("q2_k", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q2_k(w, wq2, N, K)
    del w
    X8k = torch.empty(M * q.row_bytes("q8_k", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q8_k(X, X8k, M, K)
    t2 = time_one(lambda i: q.qmm_matmul_q2_k(wq2, X8k, Y, M, N, K))
    m2_ms = t2["mean"]
    log(f"prefill q2_k weights: matmul {m2_ms * 1e3:.1f} us (median {t2['median'] * 1e3:.1f})")
    del wq2
    # Q4_K weights x Q8_K activations (the format of q4_K_M files; weights of the Q4_K workload)
    w = torch.from_numpy(synth.weights(N, K, config=5)).cuda()
    wq4k = torch.empty(N * q.row_bytes("q4_k", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q4_k(w, wq4k, N, K)
    del w
    t4 = time_one(lambda i: q.qmm_matmul_q4_k(wq4k, X8k, Y, M, N, K))
    m4_ms = t4["mean"]
    log(f"prefill q4_k weights: matmul {m4_ms * 1e3:.1f} us (median {t4['median'] * 1e3:.1f})")
    del wq4k
    # Q6_K weights x Q8_K activations (weights of the Q6_K workload)
    w = torch.from_numpy(synth.weights(N, K, config=6)).cuda()
    wq6k = torch.empty(N * q.row_bytes("q6_k", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q6_k(w, wq6k, N, K)
    del w
    t6 = time_one(lambda i: q.qmm_matmul_q6_k(wq6k, X8k, Y, M, N, K))
    m6_ms = t6["mean"]
    log(f"prefill q6_k weights: matmul {m6_ms * 1e3:.1f} us (median {t6['median'] * 1e3:.1f})")
    del wq6k, X8k
    return dict(ms_step=ms_step, nsteps=nsteps, step_us=us(st), tops=ops / (ms_step * 1e-3) / 1e12, y_check=y_check,
                roofline={"kernel": "qmm::k_matmul_q4_0", "bound": "mfma", "achieved": round(tops_kernel, 2),
                          "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(tops_kernel / INT8_PEAK_TOPS, 4),
                          "traffic": committed_traffic("k_matmul_q4_0", "2048x12288x4096"),
                          "kernel_us_mean": round(mm["mean"] * 1e3, 2), "kernel_us": us(mm),
                          "algorithmic_ops": ops},
                q8_0_weights={"kernel": "qmm::k_matmul_q8_0", "kernel_us_mean": round(m8_ms * 1e3, 2), "kernel_us": us(t8),
                              "achieved": round(ops / (m8_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                              "frac": round(ops / (m8_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              "traffic": committed_traffic("k_matmul_q8_0", "2048x12288x4096")},
                q5_0_weights={"kernel": "qmm::k_matmul_q5_0", "kernel_us_mean": round(m5_ms * 1e3, 2), "kernel_us": us(t5),
                              "achieved": round(ops / (m5_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                              "frac": round(ops / (m5_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              "traffic": committed_traffic("k_matmul_q5_0", "2048x12288x4096")},
                q4_1_weights=off["q4_1"], q5_1_weights=off["q5_1"],
                q2_k_weights={"kernel": "qmm::k_matmul_k<Q2_K>", "kernel_us_mean": round(m2_ms * 1e3, 2), "kernel_us": us(t2),
                              "achieved": round(ops / (m2_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                              "frac": round(ops / (m2_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              "traffic": committed_traffic("k_matmul_q2_k", "2048x12288x4096")},
                q4_k_weights={"kernel": "qmm::k_matmul_k<Q4_K>", "kernel_us_mean": round(m4_ms * 1e3, 2), "kernel_us": us(t4),
                              "achieved": round(ops / (m4_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                              "frac": round(ops / (m4_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              "traffic": committed_traffic("k_matmul_q4_k", "2048x12288x4096")},
                q6_k_weights={"kernel": "qmm::k_matmul_k<Q6_K>", "kernel_us_mean": round(m6_ms * 1e3, 2), "kernel_us": us(t6),
                              "achieved": round(ops / (m6_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                              "frac": round(ops / (m6_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              "traffic": committed_traffic("k_matmul_q6_k", "2048x12288x4096")})


# The other decode workloads, one matvec launch each (and, for the formats with
# a fused entry point, the fused quantize + matvec step beside it, with no
# quantized-row output), weights rotated like the headline's: the Q8_0 set of one 7B-style layer (fused QKV and gate+up share
# the 4096-wide activation, down takes an independent 11008-wide one), Q2_K,
# the K-quants of q4_K_M files and the other 32-value formats.  (format, N, K, workload id, weight
# stream, activation stream, name); the ids seed the synthetic inputs.
MATVEC_CONFIGS = [
    ("q8_0", 12288, 4096, 2, 0, 1, "q8_0_qkv_12288x4096"),
    ("q8_0", 22016, 4096, 2, 3, 1, "q8_0_gate_up_22016x4096"),
    ("q8_0", 4096, 11008, 2, 4, 5, "q8_0_down_4096x11008"),
    ("q2_k", 12288, 4096, 3, 0, 1, "q2_k_12288x4096"),
    ("q4_k", 12288, 4096, 5, 0, 1, "q4_k_12288x4096"),
    ("q6_k", 12288, 4096, 6, 0, 1, "q6_k_12288x4096"),
    ("q4_1", 12288, 4096, 9, 0, 1, "q4_1_12288x4096"),
    ("q5_0", 12288, 4096, 10, 0, 1, "q5_0_12288x4096"),
    ("q5_1", 12288, 4096, 11, 0, 1, "q5_1_12288x4096"),
]


def bench_matvec_configs(args, torch, q, synth):
    """Kernel time and weight-stream GB/s of each matvec workload above."""
    rows = []
    for fmt, N, K, cfg, wstream, xstream, name in MATVEC_CONFIGS:
        wbytes = N * q.row_bytes(fmt, K)
        w = torch.from_numpy(synth.weights(N, K, config=cfg, stream=wstream)).cuda()
        wq0 = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
        q.QUANTIZE_W[fmt](w, wq0, N, K)
        del w
        copies = max(2, int(args.copies_mb * 1e6 // wbytes) + 1)
        wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
        x = torch.from_numpy(synth.activations(1, K, config=cfg, stream=xstream)).cuda()
        act = q.ACT_FORMAT[fmt]
        xq = torch.empty(q.row_bytes(act, K), dtype=torch.uint8, device="cuda")
        q.QUANTIZE_X[fmt](x, xq, 1, K)
        y = torch.empty(N, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        mv = q.MATVEC[fmt]
        launches = [lambda i: mv(wqs[i % copies], xq, y, N, K)]
        fz = q.QUANTIZE_MATVEC.get(fmt)
        if fz is not None:
            # the decode step from the f32 activation: one fused launch
            launches.append(lambda i: fz(wqs[i % copies], x, None, y, N, K))
        ts = time_kernels(torch, launches, copies, max(200, args.steps))
        t = ts[0]
        ms = t["mean"]
        gbs = wbytes / (ms * 1e-3) / 1e9
        log(f"matvec {name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM) over "
            f"{copies} weight copies" + (f"; fused step {ts[1]['mean'] * 1e3:.2f} us" if fz is not None else ""))
        row = {"workload": name, "format": fmt, "N": N, "K": K, "weight_bytes": wbytes,
               "kernel_us_mean": round(ms * 1e3, 3), "kernel_us": us(t),
               "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if fz is not None:
            row["fused_step_us_mean"] = round(ts[1]["mean"] * 1e3, 3)
            row["fused_step_us"] = us(ts[1])
        rows.append(row)
        del wqs, wq0
        torch.cuda.empty_cache()
    # embedding rows: 2048 token ids into a Q4_0 table of 151936 x 896 (the
    # vocabulary shape of the 0.5B model the pages measure)
    Nt, Kt, nid = 151936, 896, 2048
    tb = Nt * q.row_bytes("q4_0", Kt)
    w = torch.from_numpy(synth.weights(Nt, Kt, config=7)).cuda()
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q4_0(w, table, Nt, Kt)
    del w
    ids = torch.from_numpy((synth.splitmix64(synth.seed_for(7, 1), 0, nid) % Nt).astype("int32")).cuda()
    emb = torch.empty((nid, Kt), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t = time_kernels(torch, [lambda i: q.qmm_get_rows_q4_0(table, ids, emb, nid, Nt, Kt)], 20, max(200, args.steps))[0]
    ms = t["mean"]
    moved = nid * (q.row_bytes("q4_0", Kt) + 4 * Kt + 4)
    gbs = moved / (ms * 1e-3) / 1e9
    log(f"get_rows q4_0 {nid} of {Nt}x{Kt}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s of rows read + written")
    rows.append({"workload": f"q4_0_get_rows_{nid}_of_{Nt}x{Kt}", "format": "q4_0", "N": Nt, "K": Kt,
                 "ids": nid, "bytes_moved": moved, "kernel_us_mean": round(ms * 1e3, 3),
                 "kernel_us": us(t), "achieved_gbs": round(gbs, 1),
                 "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    del table
    layer = [r for r in rows if r["workload"].startswith("q8_0_")]
    tot_b = sum(r["weight_bytes"] for r in layer)
    tot_us = sum(r["kernel_us_mean"] for r in layer)
    return {"unit": "GB/s", "bound": "hbm", "peak": HBM_PEAK_GBS, "rows": rows,
            "q8_0_layer_sum": {"weight_bytes": tot_b, "kernel_us": round(tot_us, 3),
                               "achieved_gbs": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                               "hbm_frac": round(tot_b / (tot_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}


def bench_peaks(args, torch, q, sizes=()):
    """Measured ceilings (the probes of libqmm_probe.so).  Reads: every
    configuration of the read probe (1, 2, 4, 8, 16 loads in flight per lane;
    4, 8, 16 waves per workgroup; plain or non-temporal loads) over passes of
    the decode's 28,311,552 weight bytes, each launch on the next of 37
    rotating slices of a 1 GiB buffer (> the 256 MB last-level cache, so each
    pass is cold, as each decode step is), timed like the kernels they bound;
    the fastest is the attainable 28 MB read, and the same configuration
    gives a 1 GiB pass and a pass of every other decode workload's weight
    size in `sizes`.  MFMA: back-to-back int8 MFMAs on register operands at
    two and three waves per SIMD.  Issue: f32 FMAs (vector-register operands,
    as in the prefill folds), int8 MFMAs, both interleaved, and the FMAs with a
    scalar operand, at two waves per SIMD: the vector-ALU cost of an FMA and
    the FMA issue time an MFMA takes when both run."""
    from matmul_quantize_q8_amd import probe
    size = 1 << 30
    buf = torch.arange(size // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(size // 16384 + 1, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    S = DEC["N"] * q.row_bytes("q4_0", DEC["K"])
    ns = size // S
    configs = [(lpl, nw, nt) for nt in (True, False) for nw in probe.WAVES_PER_WG for lpl in probe.LOADS_PER_LANE
               if probe.read_span(lpl, nw) >= 16384]

    def launcher(B, lpl, nw, nt):
        nsl = size // B
        return lambda i: probe.qmm_peak_read(base + (i % nsl) * B, B, sink, lpl, nw, nt)

    sweep = time_kernels(torch, [launcher(S, *c) for c in configs], ns, max(2 * ns, 74), warm_ms=25.0)
    best = min(range(len(configs)), key=lambda k: sweep[k]["mean"])
    bl, bw, bn = configs[best]
    sl = sweep[best]
    big = time_kernels(torch, [lambda i: probe.qmm_peak_read(base, size, sink, bl, bw, bn)], 4, 24)[0]
    by_size = {}
    for B in sorted(set(sizes)):
        tb = time_kernels(torch, [launcher(B, bl, bw, bn)], size // B, max(2 * (size // B), 74), warm_ms=5.0)[0]
        by_size[str(B)] = round(tb["mean"] * 1e3, 3)
    del buf
    mfma = []
    for wg, iters in ((512, 4000), (768, 2700)):
        out = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
        probe.qmm_peak_mfma_i8(out, wg, iters)
        torch.cuda.synchronize()
        if not bool((out == 2048 * iters).all()):
            raise RuntimeError("int8 MFMA probe returned wrong sums")
        tm = time_kernels(torch, [lambda i: probe.qmm_peak_mfma_i8(out, wg, iters)], 2, 8)[0]
        ops = wg * 4 * 4 * iters * 2.0 * 32 * 32 * 32
        mfma.append((ops / (tm["mean"] * 1e-3) / 1e12, wg * 4 // 1024, tm["mean"]))   # 4 waves per workgroup, 1024 SIMDs
    tops, waves, mms = max(mfma)
    # issue rates at two waves per SIMD (the prefill kernels' occupancy): f32
    # FMAs with vector-register operands (the folds' form) alone, int8 MFMAs
    # alone, both interleaved, and the FMAs with one scalar operand; clocks at
    # 2.4 GHz
    it, wps = 2000, 2
    n = 256 * 256 * wps
    fo = torch.empty(n, dtype=torch.float32, device="cuda")
    io = torch.empty(n, dtype=torch.int32, device="cuda")
    modes = ("fma", "mfma", "mixed", "fma_sgpr")
    for mode in modes:
        probe.qmm_probe_issue(mode, wps, it, fo, io)
        torch.cuda.synchronize()
        if not bool((io == (0 if mode.startswith("fma") else 2048 * it)).all()) or not bool(torch.isfinite(fo).all()):
            raise RuntimeError(f"issue probe ({mode}) returned wrong results")
    ti = time_kernels(torch, [lambda i, m=m: probe.qmm_probe_issue(m, wps, it, fo, io) for m in modes], 2, 8)
    t_fma, t_mfma, t_mix, t_sg = (t["mean"] * 1e-3 for t in ti)
    n_fma, n_mfma = wps * it * 128, wps * it * 4          # per SIMD
    issue = {"waves_per_simd": wps, "iters": it,
             "us": {m: round(t * 1e6, 2) for m, t in zip(modes, (t_fma, t_mfma, t_mix, t_sg))},
             "clk_per_fma": round(t_fma * 2.4e9 / n_fma, 3), "clk_per_fma_sgpr_operand": round(t_sg * 2.4e9 / n_fma, 3),
             "clk_per_mfma": round(t_mfma * 2.4e9 / n_mfma, 2),
             "fma_clk_taken_per_mfma_when_mixed": round((t_mix - t_fma) * 2.4e9 / n_mfma, 2),
             "mfma_time_hidden_frac": round(1.0 - (t_mix - t_fma) / t_mfma, 3),
             "clock_assumed_ghz": 2.4}
    del fo, io
    res = {"hbm_read_1GiB_gbs": round(size / (big["mean"] * 1e-3) / 1e9, 1),
           "hbm_read_28MB_gbs": round(S / (sl["mean"] * 1e-3) / 1e9, 1),
           "hbm_read_28MB_us": us(sl),
           "hbm_read_best": {"loads_per_lane": bl, "waves_per_wg": bw, "nontemporal": bn},
           "hbm_read_28MB_sweep_us": {f"lpl{c[0]}_w{c[1]}_{'nt' if c[2] else 'plain'}": round(t["mean"] * 1e3, 3)
                                      for c, t in zip(configs, sweep)},
           "hbm_read_us_by_bytes": by_size,
           "int8_mfma_tops": round(tops, 1), "int8_mfma_waves_per_simd": waves,
           "issue": issue,
           "kernels": ["qmm::k_probe_read", "qmm::k_peak_mfma_i8", "qmm::k_probe_issue"]}
    log(f"peaks: read 1 GiB {res['hbm_read_1GiB_gbs']} GB/s, 28 MB passes {res['hbm_read_28MB_gbs']} GB/s "
        f"({sl['mean'] * 1e3:.2f} us, best of {len(configs)}: {bl} loads/lane, {bw} waves, "
        f"{'non-temporal' if bn else 'plain'}), int8 MFMA {tops:.0f} TOPS at {waves} waves/SIMD; "
        f"issue: {issue['clk_per_fma']} clk/FMA ({issue['clk_per_fma_sgpr_operand']} with a scalar operand), "
        f"{issue['clk_per_mfma']} clk/MFMA, mixed: "
        f"{issue['fma_clk_taken_per_mfma_when_mixed']} FMA clk per MFMA")
    return res


def bench_few_tokens(args, torch, q, synth):
    """qmm_matmul_* for a few tokens (M = 2 ... 128) at 12288 x 4096, Q4_0 and
    Q4_K weights (the decode workloads' weights, rotated over copies like the
    decode bench): kernel time, and the time of M decode launches beside it."""
    N, K = DEC["N"], DEC["K"]
    rows = []
    for fmt, cfg in (("q4_0", 1), ("q4_k", 5)):
        w = torch.from_numpy(synth.weights(N, K, config=cfg)).cuda()
        wbytes = N * q.row_bytes(fmt, K)
        wq0 = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
        q.QUANTIZE_W[fmt](w, wq0, N, K)
        del w
        copies = max(2, int(args.copies_mb * 1e6 // wbytes) + 1)
        wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
        for M in (2, 8, 16, 32, 64, 128):
            x = torch.from_numpy(synth.activations(M, K, config=cfg)).cuda()
            xq = torch.empty(M * q.row_bytes(q.ACT_FORMAT[fmt], K), dtype=torch.uint8, device="cuda")
            q.QUANTIZE_X[fmt](x, xq, M, K)
            y = torch.empty(M * N, dtype=torch.float32, device="cuda")
            tm, tv = time_kernels(torch, [lambda i: q.MATMUL[fmt](wqs[i % copies], xq, y, M, N, K),
                                          lambda i: q.MATVEC[fmt](wqs[i % copies], xq, y, N, K)],
                                  copies, max(2 * copies, args.steps), warm_ms=10.0)
            ms, mv = tm["mean"], tv["mean"]
            log(f"few tokens {fmt} M={M}: {ms * 1e3:.2f} us ({M} decode launches {M * mv * 1e3:.2f} us)")
            rows.append({"format": fmt, "M": M, "N": N, "K": K, "kernel_us_mean": round(ms * 1e3, 3),
                         "kernel_us": us(tm),
                         "tops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 3),
                         "m_decode_launches_us": round(M * mv * 1e3, 3)})
        del wqs, wq0
        torch.cuda.empty_cache()
    return rows


def cpu_threads():
    """Threads for the oracle: every core this process may run on, capped by
    OMP_NUM_THREADS when the host sets it (a shared host's CPU share for this
    job), and the host's logical CPU count beside it."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n), os.cpu_count()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def output_check(y, ref):
    """The benchmarked outputs y against the oracle's exact values and term
    magnitudes (ref from oracle.matmul with want=("y64", "mag"))."""
    import numpy as np
    y64, mag = ref["y64"].reshape(y.shape), ref["mag"].reshape(y.shape)
    worst = float(np.max(np.abs(y.astype(np.float64) - y64) / (TOL * np.maximum(mag, 1e-300))))
    return {"outputs": int(y.size), "bound": f"|y - exact| <= {TOL:g} * sum of |terms| per output",
            "max_err_over_bound": round(worst, 4), "ok": bool(worst <= 1.0)}


def cpu_baseline_decode(args, q, synth, y_gpu=None):
    import oracle
    N, K = DEC["N"], DEC["K"]
    w = synth.weights(N, K, config=1)
    x = synth.activations(1, K, config=1, outlier_frac=0.01, outlier_factor=20.0)
    wq = oracle.quantize_q4_0_w(w)
    thr, host = cpu_threads()
    reps, t_total = 0, 0.0
    while t_total < args.cpu_seconds or reps < 1:
        t = time.perf_counter()
        xq = oracle.quantize_q8_0(x)
        oracle.matmul("q4_0", wq, xq, 1, N, K, threads=thr, want=("y",))
        t_total += time.perf_counter() - t
        reps += 1
    per = t_total / reps
    # the scalar oracle on one core, over a quarter of the budget
    reps1, t1 = 0, 0.0
    while t1 < args.cpu_seconds / 4 or reps1 < 1:
        t = time.perf_counter()
        xq = oracle.quantize_q8_0(x)
        oracle.matmul("q4_0", wq, xq, 1, N, K, threads=1, want=("y",))
        t1 += time.perf_counter() - t
        reps1 += 1
    per1 = t1 / reps1
    res = {"value": round(wq.nbytes / per / 1e9, 3), "unit": "GB/s", "cores": thr, "kind": "oracle",
           "sample": f"full {N}x{K} decode step (quantize + matvec), {reps} repeats, {per * 1e3:.1f} ms each",
           "host_logical_cpus": host, "cpu_model": cpu_model(),
           "single_core": {"value": round(wq.nbytes / per1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"the same step, {reps1} repeats, {per1 * 1e3:.1f} ms each"}}
    if y_gpu is not None:   # untimed: the benchmarked step's output against the oracle
        ref = oracle.matmul("q4_0", wq, oracle.quantize_q8_0(x), 1, N, K, threads=thr, want=("y64", "mag"))
        res["output_check"] = output_check(y_gpu, ref)
        log(f"decode output check: {res['output_check']}")
    return res


def cpu_baseline_prefill(args, q, synth, y_gpu=None):
    """The whole 2048-token prefill (quantize + product) on all the threads,
    and the scalar oracle on one core over the first 64 tokens, extrapolated
    to 2048 (the product's cost is linear in the token count)."""
    import oracle
    M, N, K = PRE["M"], PRE["N"], PRE["K"]
    w = synth.weights(N, K, config=1)
    wq = oracle.quantize_q4_0_w(w)
    thr, host = cpu_threads()
    x = synth.activations(M, K, config=4)
    t = time.perf_counter()
    xq = oracle.quantize_q8_0(x)
    oracle.matmul("q4_0", wq, xq, M, N, K, threads=thr, want=("y",))
    dt = time.perf_counter() - t
    m1 = 64
    t = time.perf_counter()
    xq1 = oracle.quantize_q8_0(x[:m1])
    oracle.matmul("q4_0", wq, xq1, m1, N, K, threads=1, want=("y",))
    dt1 = time.perf_counter() - t
    ops = 2.0 * M * N * K
    res = {"value": round(ops / dt / 1e12, 5), "unit": "TOPS", "cores": thr, "kind": "oracle",
            "sample": f"all {M} tokens of the {M}x{N}x{K} prefill ({dt:.1f} s)",
            "host_logical_cpus": host, "cpu_model": cpu_model(),
            "single_core": {"value": round(2.0 * m1 * N * K / dt1 / 1e12, 6), "unit": "TOPS", "cores": 1,
                            "sample": f"first {m1} of {M} tokens ({dt1:.1f} s), extrapolated to {M}: "
                                      f"{dt1 * M / m1:.0f} s"}}
    if y_gpu is not None:   # untimed: the benchmarked step's first rows against the oracle
        r = y_gpu.shape[0]
        ref = oracle.matmul("q4_0", wq, oracle.quantize_q8_0(x[:r]), r, N, K, threads=thr, want=("y64", "mag"))
        res["output_check"] = output_check(y_gpu, ref)
        log(f"prefill output check ({r} token rows): {res['output_check']}")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the kernels run on one "
              "MI355X; sharding the weight rows over several GPUs is a documented design, not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import matmul_quantize_q8_amd as q
    import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    q.lib()
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}")
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n}), flush=True)
        return

    sizes = [N * q.row_bytes(fmt, K) for fmt, N, K, *_ in MATVEC_CONFIGS] if args.only in ("all", "configs") else []
    peaks = None if args.skip_peaks else bench_peaks(args, torch, q, sizes)
    dec = bench_decode(args, torch, q, synth) if args.only in ("all", "decode") else None
    small = bench_small(args, torch, q, synth) if args.only in ("all", "decode") else None
    pre = bench_prefill(args, torch, q, synth) if args.only in ("all", "prefill") else None
    cfgs = bench_matvec_configs(args, torch, q, synth) if args.only in ("all", "configs") else None
    few = bench_few_tokens(args, torch, q, synth) if args.only in ("all", "configs") else None

    cpu_dec = cpu_pre = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host cores")
        if dec is not None:
            cpu_dec = cpu_baseline_decode(args, q, synth, dec["y_check"])
        if pre is not None:
            cpu_pre = cpu_baseline_prefill(args, q, synth, pre["y_check"])

    out = {"metric": METRIC, "n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "int8", "data": "synthetic"}
    if dec is not None and peaks is not None:
        dec["roofline"]["frac_of_attainable"] = round(peaks["hbm_read_28MB_us"]["mean"] / dec["roofline"]["kernel_us_mean"],
                                                      4)
    if pre is not None and peaks is not None:
        pre["roofline"]["frac_of_attainable"] = round(pre["roofline"]["achieved"] / peaks["int8_mfma_tops"], 4)
    if dec is not None:
        out.update({"value": round(dec["gbs"], 1), "unit": "GB/s", "steps": dec["nsteps"], "warmup": args.warmup,
                    "ms_per_step": round(dec["ms_step"], 5),
                    "config": {"workload": "q4_0_matvec_12288x4096", "M": 1, "N": DEC["N"], "K": DEC["K"],
                               "weight_bytes": dec["wbytes"], "weight_copies": dec["copies"],
                               "step": "quantize_matvec_q4_0 (quantize + matvec in one launch), replayed "
                                       "from HIP graphs after a warm-up",
                               "hbm_frac_step": round(dec["gbs"] / HBM_PEAK_GBS, 4),
                               "ms_per_step_eager_python": round(dec["ms_step_eager"], 5),
                               "ms_per_step_two_launches": round(dec["ms_two"], 5)},
                    "roofline": dec["roofline"], "cpu_baseline": cpu_dec})
    if small is not None:
        out["small_and_quantizers"] = small
    if pre is not None:
        pf = {"workload": "q4_0_matmul_2048x12288x4096", "value": round(pre["tops"], 2), "unit": "TOPS",
              "steps": pre["nsteps"], "warmup": args.prefill_warmup, "ms_per_step": round(pre["ms_step"], 4),
              "step_us": pre["step_us"],
              "step_ge_kernel": pre["ms_step"] >= pre["roofline"]["kernel_us_mean"] * 1e-3,
              "step": "quantize_q8_0 (2048x4096) + matmul_q4_0, graphs of 4 steps alternating with graphs of "
                      "4 matmuls in the same rounds", "roofline": pre["roofline"],
              "q8_0_weights": pre["q8_0_weights"], "q2_k_weights": pre["q2_k_weights"],
              "q5_0_weights": pre["q5_0_weights"], "q4_1_weights": pre["q4_1_weights"],
              "q5_1_weights": pre["q5_1_weights"], "q4_k_weights": pre["q4_k_weights"],
              "q6_k_weights": pre["q6_k_weights"], "cpu_baseline": cpu_pre}
        if dec is None:
            out.update({"value": pf["value"], "unit": "TOPS", "steps": pf["steps"], "warmup": pf["warmup"],
                        "ms_per_step": pf["ms_per_step"], "config": {"workload": pf["workload"]},
                        "roofline": pf["roofline"], "cpu_baseline": cpu_pre})
        else:
            out["prefill"] = pf
    if cfgs is not None:
        for r in cfgs["rows"]:
            att = peaks["hbm_read_us_by_bytes"].get(str(r.get("weight_bytes"))) if peaks is not None else None
            if att is not None:
                r["attainable_read_us"] = att
                r["frac_of_attainable"] = round(att / r["kernel_us_mean"], 4)
        out["matvec_configs"] = cfgs
    if few is not None:
        out["few_tokens"] = few
    if peaks is not None:
        out["attainable"] = peaks
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
