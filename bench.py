"""Benchmark of the W6A6 / W6A8 linear-layer path on LLaMA-2-70B shapes, one MI355X.

A step is one pass of the hot path over one batch of synthetic input: for every
token count M in {1, 16, 64, 256, 1024, 4096}, both activation precisions (A6, A8)
and the four linear layers of a LLaMA-2-70B decoder block (qkv 10240x8192,
o 8192x8192, gate_up 57344x8192, down 8192x28672), quantize the fp16 activations
(flexq_quant_act) and run the W6Ax GEMM on packed 6-bit weights resident in HBM:
flexq_gemm_w6ax with its automatic kernel choice, or flexq_gemm_w6ax_splitk in the
planned configuration where flexq_gemm_w6ax_splitk_plan cuts K into slices (mid-sized
M on the narrow layers); where the choice is the weight-streaming kernel the codes are
quantized into and read from 16-row blocks (flexq_quant_act_blocked,
flexq_gemm_w6ax_blocked).  Weights are packed once, before timing (offline step).

Prints one JSON line: value = whole-step GEMM+quant throughput in TOPS (2*M*N*K
integer ops per GEMM, M unpadded), per-shape TOPS / GB/s / roofline fractions,
the roofline of the dominant kernel, on-device peak measurements and the CPU
oracle timed on a bounded sample.  The step is captured once as a HIP graph whose
replays give ms_per_step and value (--eager: the launch-by-launch step instead).
Per-kernel figures come from runs of --reps back-to-back launches of each shape
between HIP events (the GEMM rotating over weight copies so none is served from
the Infinity Cache), medians and p10 / p90 over --steps runs.
--summarize-trace DB turns a rocprofv3 kernel trace of such a run into the
markdown tables kept under profiles/, with the same figures recomputed from the
kernel durations.  --power SECONDS reports board power and shader clock (amd-smi)
under the prefill GEMM and the on-device peak loops instead of running the step.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "W6A6/W6A8 GEMM TOPS + HBM GB/s (% roofline), LLaMA-2-70B linear shapes"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
GROUP = 128
LAYERS = synth.LLAMA2_70B
# one GPU's share of the same layers under 8-way tensor parallelism: qkv and gate_up
# split along N, o and down along K at whole 128-groups
LAYERS_TP8 = {"qkv": (10240 // 8, 8192), "o": (8192, 8192 // 8),
              "gate_up": (57344 // 8, 8192), "down": (8192, 28672 // 8)}
WORKLOAD_NAMES = {"70b": "llama2_70b_linear_layers_w6a6_w6a8",
                  "70b_tp8": "llama2_70b_tp8_shard_linear_layers_w6a6_w6a8",
                  "70b_stack": "llama2_70b_80_layer_stack_w6a6_w6a8"}
STACK_LAYERS, STACK_A8_LAYERS, STACK_M = 80, 8, (32, 2048)
M_LIST = (1, 16, 64, 256, 1024, 4096)
ABITS = (6, 8)


TILE_NAMES = {3: "256x128", 4: "128x128", 5: "128x64", 7: "64x128"}
REPS_IN_RUN = 20   # back-to-back launches per timed run of one shape


def gemm_bytes(M, N, K):
    """Algorithmic HBM bytes of one GEMM: packed W + fp16 s_w + int8 q_a + fp32 s_a + fp16 Y."""
    G = K // GROUP
    return 0.75 * N * K + 2 * N * G + M * K + 4 * M * G + 2 * M * N


def quant_bytes(M, K):
    """fp16 X in, int8 q_a + fp32 s_a out."""
    return 2 * M * K + M * K + 4 * M * (K // GROUP)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--seed", type=int, default=synth.BASE_SEED)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the on-device peak measurements (HBM read, MFMA loop)")
    p.add_argument("--eager", action="store_true",
                   help="time the step launch by launch only (no HIP graph replay)")
    p.add_argument("--cpu-sample-cols", type=int, default=512,
                   help="output columns per GEMM in the oracle's timed sample")
    p.add_argument("--m", type=str, default=None, help="comma list overriding the token counts")
    p.add_argument("--layers", choices=sorted(WORKLOAD_NAMES), default="70b",
                   help="70b: the LLaMA-2-70B linear layers (the benchmark's workload); "
                        "70b_tp8: one GPU's share of them under 8-way tensor parallelism; "
                        "70b_stack: all 80 decoder layers resident (52 GB packed), a decode "
                        "pass at M = 32 and a prefill pass at M = 2048, A8 on 8 seeded layers")
    p.add_argument("--reps", type=int, default=REPS_IN_RUN,
                   help="back-to-back launches per timed run of one shape (fewer for "
                        "counter-collection runs, where every launch is profiled)")
    p.add_argument("--summarize-trace", metavar="DB", default=None,
                   help="print a markdown summary of a rocprofv3 --kernel-trace database of a "
                        "bench run (per-kernel times, GEMM launches by grid, the prefill "
                        "kernel's int8 fraction recomputed from the trace) and exit")
    p.add_argument("--a6-packed", action="store_true",
                   help="also compare, at every M <= 64 and layer, the streaming GEMM over one "
                        "byte per A6 code with flexq_gemm_w6a6_packed over 6-bit codes, and the "
                        "two activation quantizers (key a6_packed)")
    p.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                   help="instead of the step: board power and shader clock (amd-smi) while "
                        "the prefill GEMM (70B gate_up, M = 4096), the rescale loop, the "
                        "MFMA-only loop and a plain HBM read each run back to back for "
                        "SECONDS; one JSON line, then exit")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="first run one device-to-device copy of this many MiB (the known-size "
                        "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_prefill_llama2_70b.md")
PREFILL_SRC = os.path.join(ROOT, "w6a6_w6a8_integer_amd", "csrc", "gemm_prefill.hip")


def recorded_traffic():
    """HBM bytes per prefill launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a copy kernel of known size), as recorded next to the hash
    of the kernel source it was taken on; None once that source has changed."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        src = hashlib.sha256(open(PREFILL_SRC, "rb").read()).hexdigest()
    except OSError:
        return None
    rec = {}
    for line in text.splitlines():
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_sha256") != src:
        return None
    try:
        return int(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_kind(fq, M, N, K):
    """How the step runs one GEMM: ("splitk", S, tile path) where the split-K plan
    cuts K, else ("decode",) or ("prefill",) as flexq_gemm_w6ax's automatic choice."""
    S, tile = fq.splitk_plan(M, N, K)
    if S > 1:
        return ("splitk", S, tile)
    return ("decode",) if fq.auto_path(M, N, K) == fq.PATH_DECODE else ("prefill",)


def kernel_label(kind, M, N, K, fq):
    if kind[0] == "splitk":
        return f"splitk {TILE_NAMES[kind[2]]} x{kind[1]}"
    if kind[0] == "decode":
        return "decode"
    return TILE_NAMES[fq.prefill_tile(M, N, K)] + ("+128x64" if fq.prefill_main_cols(M, N, K) < N
                                                   else "")


def summarize_trace(db, layers, m_list, reps):
    """Markdown summary of a rocprofv3 kernel-trace database (the `kernels` view of
    its SQLite output) of a bench run on `layers` at token counts `m_list`."""
    import sqlite3
    import w6a6_w6a8_integer_amd as fq
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration, grid_x, workgroup_x from kernels").fetchall()
    print("| kernel | calls | total (us) | average (us) | share % |\n|---|---|---|---|---|")
    tot = sum(r[1] for r in rows)
    agg = {}
    for name, dur, gx, wx in rows:
        a = agg.setdefault(name, [0, 0.0])
        a[0] += 1
        a[1] += dur
    for name, (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"| `{name[:90]}` | {n} | {t / 1e3:.1f} | {t / n / 1e3:.2f} | {100 * t / tot:.2f} |")
    # GEMM launches by (kernel, grid): prefill launches matched to their shapes by tile
    # and grid (the tail split's two kernels per call both counted)
    grids = {}
    for name, dur, gx, wx in rows:
        if "gemm_" in name or "splitk_reduce" in name:
            g = grids.setdefault((name, gx // max(wx, 1)), [])
            g.append(dur)
    print("\n| kernel | workgroups | calls | avg (us) | min (us) | max (us) |\n|---|---|---|---|---|---|")
    for (name, wg), d in sorted(grids.items()):
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        print(f"| `{short}` | {wg} | {len(d)} | {sum(d) / len(d) / 1e3:.2f} | {min(d) / 1e3:.2f} "
              f"| {max(d) / 1e3:.2f} |")
    # The per-kernel runs of the bench, recognized in dispatch order: a busy kernel,
    # REPS_IN_RUN quantizer launches, then the GEMM launches of one (M, abits, layer)
    # (two kernels per call where the prefill tail split applies or split-K adds its
    # reduce); runs come in the
    # bench's shape order, `steps` times over.
    ordered = con.execute("select name, duration from kernels order by start").fetchall()
    keys = sorted({(M, ab, n) for M in m_list for ab in ABITS for n in layers},
                  key=lambda k: (-k[0], k[1], list(layers).index(k[2])))
    runs, i = [], 0
    while i < len(ordered):
        if "peak_mfma_kernel" in ordered[i][0]:
            j = i + 1
            nq = 0
            while j < len(ordered) and "quant_act_kernel" in ordered[j][0]:
                j += 1
                nq += 1
            g = []
            while j < len(ordered) and ("gemm_" in ordered[j][0] or
                                        "splitk_reduce" in ordered[j][0]):
                g.append(ordered[j][1])
                j += 1
            if nq == reps and g:
                runs.append(g)
            i = j
        else:
            i += 1
    if not runs or len(runs) % len(keys):
        print(f"\n{len(runs)} per-kernel runs found; expected a multiple of {len(keys)}")
        return
    per_key = {k: [] for k in keys}
    for r, g in enumerate(runs):
        per_key[keys[r % len(keys)]].append(sum(g) / reps)   # ns per call
    pre_ops = pre_ns = dec_b = dec_ns = 0.0
    print("\n| layer | M | abits | kernel | trace us per call (median of runs) |\n|---|---|---|---|---|")
    for k in sorted(keys, key=lambda k: (k[0], k[1], list(layers).index(k[2]))):
        M, ab, name = k
        N, K = layers[name]
        t = statistics.median(per_key[k])
        kind = gemm_kind(fq, M, N, K)
        dec = kind[0] == "decode"
        print(f"| {name} | {M} | {ab} | {kernel_label(kind, M, N, K, fq)} | {t / 1e3:.2f} |")
        if dec and M <= 16:
            dec_b += gemm_bytes(M, N, K)
            dec_ns += t
        if kind[0] == "prefill":
            pre_ops += 2.0 * M * N * K
            pre_ns += t
    if pre_ns:
        tops = pre_ops / (pre_ns * 1e-9) / 1e12
        print(f"\nFrom the trace: prefill {tops:.1f} TOP/s = {tops / INT8_PEAK_TOPS:.4f} of "
              f"{INT8_PEAK_TOPS:.0f} (the bench's roofline.frac), "
              f"M >= 1024 only: see the rows above; decode at M <= 16: "
              f"{dec_b / (dec_ns * 1e-9) / 1e9:.1f} GB/s = "
              f"{dec_b / (dec_ns * 1e-9) / 1e9 / HBM_PEAK_GBS:.4f} of {HBM_PEAK_GBS:.0f} "
              f"(the bench's hbm_frac_m_le_16); {len(runs)} runs of {reps} calls")


def main():
    global LAYERS
    args = parse()
    if args.summarize_trace:
        m_list = tuple(int(v) for v in args.m.split(",")) if args.m else M_LIST
        summarize_trace(args.summarize_trace, LAYERS_TP8 if args.layers == "70b_tp8" else LAYERS,
                        m_list, args.reps)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding over GPUs is designed, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import w6a6_w6a8_integer_amd as fq

    if args.layers == "70b_tp8":
        LAYERS = LAYERS_TP8
    fq.lib()
    dev = torch.device("cuda:0")
    if args.power:
        print(json.dumps(power_profile(fq, torch, dev, args.power, args.seed)), flush=True)
        return
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")
        del src, dst
    stack = args.layers == "70b_stack"
    m_list = tuple(int(v) for v in args.m.split(",")) if args.m else (STACK_M if stack else M_LIST)
    nthreads = synth.default_threads()
    # the stack's A8 layers: a seeded choice of STACK_A8_LAYERS of the 80 (all four
    # linears of such a layer take 8-bit activations)
    a8_layers = set(np.random.default_rng(synth.derive_seed(args.seed, "stack-a8") & 0xFFFFFFFF)
                    .choice(STACK_LAYERS, STACK_A8_LAYERS, replace=False).tolist()) if stack else set()

    # ---- weights: generated on the host, packed on the GPU.  Resident copies are
    # rotated so that no layer is served from the 256 MB MALL: every (M, abits) block
    # of the step (one launch per linear layer) reads copy `block % ncopies`, so
    # consecutive blocks read different copies and a copy is read again only after
    # min(ncopies, blocks per step) - 1 other blocks, i.e. at least one other whole
    # layer set (641.7 MB for the 70B layers) has streamed through.
    t0 = time.time()
    packed = {}
    set_bytes = sum(0.75 * N * K for N, K in LAYERS.values())
    ncopies = max(2, -(-(1 << 30) // int(set_bytes)))
    if stack:
        ncopies = STACK_LAYERS  # one resident copy per decoder layer (same synthetic values)
    # The per-kernel runs launch one layer back to back: each layer gets enough copies
    # that a copy returns only after at least 1.2 GB of its other copies.
    for li, (name, (N, K)) in enumerate(LAYERS.items()):
        w = synth.weights(synth.derive_seed(args.seed, "70b", name, "w"), N, K, nthreads=nthreads)
        wd = torch.from_numpy(w).to(dev)
        del w
        copies = []
        for c in range(max(ncopies, -(-int(1.2e9) // int(gemm_bytes(1, N, K))))):
            copies.append(fq.pack_w6(wd))
        del wd
        packed[name] = copies
    torch.cuda.synchronize()
    log(f"weights packed ({time.time() - t0:.1f} s)")

    # ---- activations and outputs per (M, layer)
    bufs = {}
    for M in m_list:
        for name, (N, K) in LAYERS.items():
            x = synth.activations(synth.derive_seed(args.seed, "70b", name, "x", M), M, K,
                                  nthreads=nthreads)
            xd = torch.from_numpy(x).to(dev)
            kind = gemm_kind(fq, M, N, K)
            # the streaming kernel's shapes keep their codes in 16-row blocks
            qa = (torch.empty(fq.blocked_act_bytes(M, K), dtype=torch.int8, device=dev)
                  if kind[0] == "decode" else
                  torch.empty((M, K), dtype=torch.int8, device=dev))
            sa = torch.empty((K // GROUP, M), dtype=torch.float32, device=dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = (torch.empty(fq.splitk_workspace_bytes(M, N, K, kind[1]), dtype=torch.uint8,
                              device=dev) if kind[0] == "splitk" else None)
            bufs[(M, name)] = (x, xd, qa, sa, y, kind, ws)
    torch.cuda.synchronize()
    log(f"activations ready ({time.time() - t0:.1f} s)")

    # Largest M first: while the long prefill launches run, the host queues the rest of
    # the step, so the short decode launches at the end start back to back and their
    # events time the GPU, not the host's launch path.
    # Each launch: (M, abits, linear, weight copy).
    if stack:
        plan = [(M, 8 if layer in a8_layers else 6, name, layer)
                for M in sorted(m_list, reverse=True) for layer in range(STACK_LAYERS)
                for name in LAYERS]
    else:
        blocks = [(M, ab) for M in sorted(m_list, reverse=True) for ab in ABITS]
        plan = [(M, ab, name, b % ncopies) for b, (M, ab) in enumerate(blocks) for name in LAYERS]
    keys = sorted({e[:3] for e in plan}, key=lambda k: (-k[0], k[1], list(LAYERS).index(k[2])))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in plan]

    def quant(M, name, ab):
        """The activation quantization of one GEMM: into 16-row blocks for the streaming
        kernel, row-major for the others."""
        _, xd, qa, sa, _, kind, _ = bufs[(M, name)]
        if kind[0] == "decode":
            fq.quant_act_blocked(xd, ab, q_a_blk=qa, s_a=sa)
        else:
            fq.quant_act(xd, ab, q_a=qa, s_a=sa)

    def gemm(M, name, ab, wp, sw):
        """One GEMM of the step, as gemm_kind says it runs."""
        N, K = LAYERS[name]
        _, _, qa, sa, y, kind, ws = bufs[(M, name)]
        if kind[0] == "splitk":
            fq.gemm_w6ax_splitk(qa, sa, wp, sw, N, ab, splits=kind[1], path=kind[2], y=y,
                                workspace=ws)
        elif kind[0] == "decode":
            fq.gemm_w6ax_blocked(qa, sa, wp, sw, N, ab, y=y)
        else:
            fq.gemm_w6ax(qa, sa, wp, sw, N, ab, y=y)

    def step(timed: bool):
        for i, (M, ab, name, widx) in enumerate(plan):
            wp, sw = packed[name][widx]
            if timed:
                ev[i][0].record()
            quant(M, name, ab)
            if timed:
                ev[i][1].record()
            gemm(M, name, ab, wp, sw)
            if timed:
                ev[i][2].record()

    for s in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # The step launch by launch, with events around every kernel (the in-step times).
    step_gemm_ms = {k: [] for k in keys}
    step_ms = []
    torch.cuda.synchronize()
    wall0 = time.time()
    for s in range(args.steps):
        step(True)
        torch.cuda.synchronize()  # read this step's events
        for i, e in enumerate(plan):
            step_gemm_ms[e[:3]].append(ev[i][1].elapsed_time(ev[i][2]))
        step_ms.append(ev[0][0].elapsed_time(ev[-1][2]))
    wall = time.time() - wall0
    total_ms = sum(step_ms)
    ms_per_step_eager = statistics.median(step_ms)

    # Per-kernel times: every (M, abits, layer) GEMM, and its activation quantization,
    # launched REPS times back to back (the GEMM on rotating weight copies, at least
    # 1.2 GB apart), between two events; `steps` such runs give the median and
    # p10 / p90 of the time per launch.  A busy kernel (about 10 ms of MFMA work)
    # holds the GPU before each run, so the host has queued the whole run before the
    # GPU reaches it.  Events around single launches would add the inter-kernel gap
    # and the event packets (a few us) to every launch, a fifth of the small layers'
    # time.
    REPS = args.reps
    quant_ms = {k: [] for k in keys}
    gemm_ms = {k: [] for k in keys}
    sink = torch.empty(fq.peak_sink_bytes(), dtype=torch.uint8, device=dev)
    clock = torch.zeros(2, dtype=torch.int64, device=dev)
    r0, r1, r2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    wall1 = time.time()
    for s in range(args.steps):
        for k in keys:
            M, ab, name = k
            cps = packed[name]
            fq.peak_mfma_i8(80000, 0, sink, clock)
            r0.record()
            for j in range(REPS):
                quant(M, name, ab)
            r1.record()
            for j in range(REPS):
                wp, sw = cps[(s * REPS + j) % len(cps)]
                gemm(M, name, ab, wp, sw)
            r2.record()
            torch.cuda.synchronize()
            quant_ms[k].append(r0.elapsed_time(r1) / REPS)
            gemm_ms[k].append(r1.elapsed_time(r2) / REPS)
    wall += time.time() - wall1

    # The same step captured once as a HIP graph and replayed back to back: the kernels
    # and their arguments are the eager step's (the same weight copies); ms_per_step
    # and value come from these replays.
    graph_ms = None
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step(False)
            graph.replay()
            torch.cuda.synchronize()
        except RuntimeError as e:  # capture unsupported here: report the eager time
            log(f"HIP graph capture failed ({e}); value from the launch-by-launch steps")
            graph = None
        if graph is not None:
            gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            wall1 = time.time()
            for e0, e1 in gev:
                e0.record()
                graph.replay()
                e1.record()
            torch.cuda.synchronize()
            wall += time.time() - wall1
            graph_ms = [e0.elapsed_time(e1) for e0, e1 in gev]
            total_ms += gev[0][0].elapsed_time(gev[-1][1])
            torch.cuda.synchronize()

    # ---- aggregate
    keys_by_m = sorted(keys, key=lambda k: (k[0], k[1], list(LAYERS).index(k[2])))
    kernel_of = {k: bufs[(k[0], k[2])][5][0] for k in keys}
    tot_ops = sum(2.0 * e[0] * LAYERS[e[2]][0] * LAYERS[e[2]][1] for e in plan)
    per_step = {k: len(step_gemm_ms[k]) // len(step_ms) for k in keys}

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]

    # on-device measured peaks (include/flexq_peaks.h), after the timed region
    peaks = None if args.no_peaks else measure_peaks(fq, torch, dev, LAYERS)

    shapes = []
    for k in keys_by_m:
        M, ab, name = k
        N, K = LAYERS[name]
        g = statistics.median(gemm_ms[k])
        ops = 2.0 * M * N * K
        by = gemm_bytes(M, N, K)
        dec = kernel_of[k] == "decode"
        row = [name, M, ab, kernel_label(bufs[(M, name)][5], M, N, K, fq),
               round(g * 1e3, 2), round(pct(gemm_ms[k], 0.1) * 1e3, 2),
               round(pct(gemm_ms[k], 0.9) * 1e3, 2),
               round(statistics.median(step_gemm_ms[k]) * 1e3, 2),
               round(statistics.median(quant_ms[k]) * 1e3, 2),
               round(ops / (g * 1e-3) / 1e12, 1), round(by / (g * 1e-3) / 1e9, 1),
               round(by / (g * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
               round(ops / (g * 1e-3) / 1e12 / INT8_PEAK_TOPS, 3)]
        if peaks:
            # against what this GPU measurably reaches: a plain read of the layer's
            # weight bytes, or the back-to-back MFMA loop
            row.append(round(by / (g * 1e-3) / 1e9 / peaks["hbm_read_gbs"][name], 3) if dec
                       else round(ops / (g * 1e-3) / 1e12 / peaks["mfma_i8_tops"], 3))
        shapes.append(row)
    shape_cols = ["layer", "M", "abits", "kernel", "gemm_us_median", "gemm_us_p10",
                  "gemm_us_p90", "gemm_us_in_step", "quant_us_median", "tops", "gbs", "frac_hbm_8tbs",
                  "frac_int8_5pops"] + (["frac_measured_peak"] if peaks else [])

    def over(sel, kern):
        """Algorithmic bytes / ops over the time of the selected GEMMs, each counted as
        often as a step runs it, at its median time per launch."""
        ks = [k for k in keys if sel(k[0]) and kernel_of[k] == kern]
        ms = sum(per_step[k] * statistics.median(gemm_ms[k]) for k in ks)
        if not ms:
            return None
        byt = sum(per_step[k] * gemm_bytes(k[0], *LAYERS[k[2]]) for k in ks)
        ops = sum(per_step[k] * 2.0 * k[0] * LAYERS[k[2]][0] * LAYERS[k[2]][1] for k in ks)
        r = {"gbs": byt / (ms * 1e-3) / 1e9, "tops": ops / (ms * 1e-3) / 1e12, "ms": ms}
        if peaks:
            # time each launch would take at the plain-read rate of its layer's size
            ideal = sum(per_step[k] * gemm_bytes(k[0], *LAYERS[k[2]])
                        / (peaks["hbm_read_gbs"][k[2]] * 1e9) for k in ks)
            r["hbm_frac_measured"] = ideal / (ms * 1e-3)
        return r

    dec_all = over(lambda M: True, "decode")
    pre_all = over(lambda M: True, "prefill")
    split_all = over(lambda M: True, "splitk")
    dec16 = over(lambda M: M <= 16, "decode")
    pre1024 = over(lambda M: M >= 1024, "prefill")
    targets = {
        "hbm_frac_m_le_16": round(dec16["gbs"] / HBM_PEAK_GBS, 4) if dec16 else None,
        "hbm_frac_m_le_16_goal": 0.70,
        "int8_frac_m_ge_1024": round(pre1024["tops"] / INT8_PEAK_TOPS, 4) if pre1024 else None,
        "int8_frac_m_ge_1024_goal": 0.50,
    }
    if peaks and dec16:
        targets["hbm_frac_m_le_16_of_measured_read"] = round(dec16["hbm_frac_measured"], 4)
    if peaks and pre1024:
        targets["int8_frac_m_ge_1024_of_measured_mfma"] = round(
            pre1024["tops"] / peaks["mfma_i8_tops"], 4)
        targets["int8_frac_m_ge_1024_of_rescale_loop"] = round(
            pre1024["tops"] / peaks["rescale_loop_tops"], 4)

    pre_launches = sum(per_step[k] for k in keys if kernel_of[k] == "prefill")
    pre_kernels = sum(per_step[k] * (1 + (fq.prefill_main_cols(k[0], *LAYERS[k[2]]) <
                                          LAYERS[k[2]][0]))
                      for k in keys if kernel_of[k] == "prefill")
    if pre_all and (not dec_all or pre_all["ms"] >= dec_all["ms"]):
        roofline = {"kernel": "gemm_prefill_kernel", "bound": "mfma",
                    "achieved": round(pre_all["tops"], 1), "peak": INT8_PEAK_TOPS,
                    "unit": "TOP/s", "frac": round(pre_all["tops"] / INT8_PEAK_TOPS, 4),
                    # counters were taken on the default workload's launches only
                    "traffic": (recorded_traffic() if args.layers == "70b" and not args.m
                                else None),
                    "timing": (f"median over runs of {args.reps} back-to-back launches between HIP "
                               "events on the launch stream"),
                    "launches_per_step": pre_launches, "kernel_launches_per_step": pre_kernels,
                    "ops_per_launch": round(sum(2.0 * k[0] * LAYERS[k[2]][0] * LAYERS[k[2]][1]
                                                * per_step[k] for k in keys
                                                if kernel_of[k] == "prefill") / max(pre_launches, 1))}
        if peaks:
            roofline["measured_peak"] = round(peaks["mfma_i8_tops"], 1)
            roofline["frac_of_measured_peak"] = round(pre_all["tops"] / peaks["mfma_i8_tops"], 4)
            roofline["rescale_loop_tops"] = peaks["rescale_loop_tops"]
            roofline["frac_of_rescale_loop"] = round(pre_all["tops"] / peaks["rescale_loop_tops"], 4)
    elif dec_all:
        roofline = {"kernel": "gemm_decode_kernel", "bound": "hbm",
                    "achieved": round(dec_all["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dec_all["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                    "timing": (f"median over runs of {args.reps} back-to-back launches between "
                               "HIP events on the launch stream")}
    else:  # every GEMM of the chosen shapes runs split over K
        roofline = {"kernel": "gemm_prefill_kernel (split-K) + splitk_reduce_kernel",
                    "bound": "mfma", "achieved": round(split_all["tops"], 1),
                    "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                    "frac": round(split_all["tops"] / INT8_PEAK_TOPS, 4), "traffic": None,
                    "timing": (f"median over runs of {args.reps} back-to-back launches between "
                               "HIP events on the launch stream")}
    # the two target figures also as scalars of the roofline record
    roofline["hbm_frac_m_le_16"] = targets["hbm_frac_m_le_16"]
    roofline["int8_frac_m_ge_1024"] = targets["int8_frac_m_ge_1024"]
    roofline_decode = None
    if dec_all:
        roofline_decode = {"kernel": "gemm_decode_kernel", "bound": "hbm",
                           "achieved": round(dec_all["gbs"], 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(dec_all["gbs"] / HBM_PEAK_GBS, 4)}
        if peaks:
            roofline_decode["frac_of_measured_read"] = round(dec_all["hbm_frac_measured"], 4)

    ms_per_step = statistics.median(graph_ms) if graph_ms else ms_per_step_eager
    value = tot_ops / (ms_per_step * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(bufs, per_step, args.cpu_sample_cols, packed, ms_per_step, tot_ops)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.layers], "weight_copies": ncopies,
                   **({"stack_layers": STACK_LAYERS, "a8_layers": sorted(a8_layers)} if stack else {}),
                   "layers": {k: list(v) for k, v in LAYERS.items()}, "M": list(m_list),
                   "abits": list(ABITS), "group": GROUP,
                   "step": ("quant_act + gemm per (M, abits, layer); gemm = split-K where "
                            "planned; blocked codes for the streaming kernel")},
        "roofline": roofline, "cpu_baseline": cpu,
        "launch": "hip_graph" if graph_ms else "eager",
        "ms_per_step_eager": round(ms_per_step_eager, 3),
        "ms_per_step_p10_p90": ([round(pct(graph_ms, 0.1), 3), round(pct(graph_ms, 0.9), 3)]
                                if graph_ms else [round(pct(step_ms, 0.1), 3),
                                                  round(pct(step_ms, 0.9), 3)]),
        "timed_region_ms": round(total_ms, 2), "wall_s": round(wall, 2),
        "shape_cols": shape_cols, "shapes": shapes,
        # last, where a truncated tail of the line still shows them
        "peaks": peaks, "roofline_decode": roofline_decode, "targets": targets,
    }
    if split_all:
        # the split-K launches (prefill kernel on K slices + the fixed-order reduce)
        out["splitk"] = {"launches_per_step": sum(per_step[k] for k in keys
                                                  if kernel_of[k] == "splitk"),
                         "tops": round(split_all["tops"], 1), "gbs": round(split_all["gbs"], 1),
                         "ms_per_step": round(split_all["ms"], 4)}
    if args.a6_packed:
        tail = {k: out.pop(k) for k in ("peaks", "roofline_decode", "targets", "splitk")
                if k in out}
        out["a6_packed"] = a6_packed_ab(fq, torch, dev, bufs, packed, m_list, REPS)
        out.update(tail)
    print(json.dumps(out, separators=(",", ":")), flush=True)


def a6_packed_ab(fq, torch, dev, bufs, packed, m_list, reps):
    """6-bit activation storage against one byte per code, at every M <= 64 and layer
    (A6): the streaming GEMM (flexq_gemm_w6ax on FLEXQ_PATH_DECODE against
    flexq_gemm_w6a6_packed) on rotating weight copies, and the activation quantizer
    (flexq_quant_act against flexq_quant_act_a6_packed).  Each is the best of 4 runs of
    `reps` back-to-back launches, the two variants alternating, a busy kernel first;
    `same_bits` says whether the two GEMMs gave the same Y."""
    sink = torch.empty(fq.peak_sink_bytes(), dtype=torch.uint8, device=dev)
    clock = torch.zeros(2, dtype=torch.int64, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(runs):
        t = {}
        for rnd in range(4):
            for name in (list(runs) if rnd % 2 == 0 else list(runs)[::-1]):
                fq.peak_mfma_i8(400, 0, sink, clock)
                e0.record()
                for i in range(reps):
                    runs[name](i)
                e1.record()
                torch.cuda.synchronize()
                t[name] = min(t.get(name, float("inf")), e0.elapsed_time(e1) / reps * 1e3)
        return t

    gemm_rows, quant_rows = [], []
    for M in sorted(m for m in m_list if m <= 64):
        for name, (N, K) in LAYERS.items():
            xd = bufs[(M, name)][1]
            qa = torch.empty((M, K), dtype=torch.int8, device=dev)
            qp = torch.empty((M, 3 * K // 16), dtype=torch.int32, device=dev)
            sa = torch.empty((K // GROUP, M), dtype=torch.float32, device=dev)
            sap = torch.empty_like(sa)
            yb = torch.empty((M, N), dtype=torch.float16, device=dev)
            yp = torch.empty_like(yb)
            q = best({"bytes": lambda i: fq.quant_act(xd, 6, q_a=qa, s_a=sa),
                      "packed": lambda i: fq.quant_act_a6_packed(xd, q_a6p=qp, s_a=sap)})
            cps = packed[name]
            g = best({
                "bytes": lambda i: fq.gemm_w6ax(qa, sa, *cps[i % len(cps)], N, 6, y=yb,
                                                path=fq.PATH_DECODE),
                "packed": lambda i: fq.gemm_w6a6_packed(qp, sap, *cps[i % len(cps)], N, y=yp)})
            same = bool(torch.equal(yb.view(torch.int16), yp.view(torch.int16)) and
                        torch.equal(sa.view(torch.int32), sap.view(torch.int32)))
            gemm_rows.append([name, M, round(g["bytes"], 2), round(g["packed"], 2),
                              round(g["bytes"] / g["packed"], 3), same])
            quant_rows.append([name, M, round(q["bytes"], 2), round(q["packed"], 2),
                               round(q["bytes"] / q["packed"], 3)])
    cols = ["layer", "M", "us_bytes", "us_packed", "speedup"]
    return {"gemm_cols": cols + ["same_bits"], "gemm": gemm_rows, "quant_cols": cols,
            "quant": quant_rows}


def read_smi_power():
    """(socket power in W, mean gfx clock over the XCDs in MHz) from one
    `amd-smi metric -p -c --json` call, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=10)
    except (OSError, subprocess.TimeoutExpired):
        return None
    return parse_smi_power(r.stdout) if r.returncode == 0 else None


def parse_smi_power(text):
    """Socket power and mean gfx clock from amd-smi's metric JSON (first GPU), or None."""
    try:
        d = json.loads(text)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        watts = float(g["power"]["socket_power"]["value"])
        clks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        return (watts, sum(clks) / len(clks)) if clks else None
    except (ValueError, KeyError, IndexError, TypeError):
        return None


def summarize_power(samples, skip=2):
    """Per phase: the median power and clock of its samples, the first `skip` dropped
    (the readings lag a phase change by about a second).  samples: (phase, reading)."""
    by = {}
    for phase, rd in samples:
        if rd is not None:
            by.setdefault(phase, []).append(rd)
    out = {}
    for phase, rds in by.items():
        core = rds[skip:] if len(rds) > skip + 2 else rds
        out[phase] = {"watts_median": statistics.median(w for w, _ in core),
                      "gfx_mhz_median": round(statistics.median(c for _, c in core), 1),
                      "samples": len(core)}
    return out


def power_profile(fq, torch, dev, seconds, seed):
    """Board power and shader clock while each of four kernels runs back to back for
    `seconds`: the 256 x 128 prefill GEMM on the 70B gate_up layer at M = 4096 (A6,
    the recipe's X and W), the rescale loop, the MFMA-only loop and a plain read of
    1 GiB.  amd-smi is sampled from a thread of this process."""
    import threading
    N, K = LAYERS["gate_up"]
    M = 4096
    x = torch.from_numpy(synth.activations(synth.derive_seed(seed, "power", "x"), M, K)).to(dev)
    w = torch.from_numpy(synth.weights(synth.derive_seed(seed, "power", "w"), N, K,
                                       nthreads=synth.default_threads())).to(dev)
    wp, sw = fq.pack_w6(w)
    del w
    qa, sa = fq.quant_act(x, 6)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    sink = torch.empty(fq.peak_sink_bytes(), dtype=torch.uint8, device=dev)
    clock = torch.zeros(2, dtype=torch.int64, device=dev)
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    phase = ["idle"]
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append((phase[0], read_smi_power()))
            time.sleep(0.2)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(2.0)
    runs = {}
    for name, fn in (
            ("prefill_gate_up_m4096",
             lambda: fq.gemm_w6ax(qa, sa, wp, sw, N, 6, y=y, path=fq.PATH_PREFILL_256X128)),
            ("rescale_loop", lambda: fq.peak_mfma_i8_rescale(2000, sink, clock)),
            ("mfma_loop", lambda: fq.peak_mfma_i8(20000, 0, sink, clock)),
            ("hbm_read_1gib", lambda: fq.peak_hbm_read(buf, sink))):
        phase[0] = name
        t0, n = time.time(), 0
        while time.time() - t0 < seconds:
            for _ in range(8):
                fn()
            n += 8
            torch.cuda.synchronize()
        runs[name] = {"launches": n, "seconds": round(time.time() - t0, 2)}
        phase[0] = "after_" + name
        time.sleep(1.0)
    stop.set()
    th.join()
    phases = summarize_power(samples)
    for name, r in runs.items():
        phases.setdefault(name, {}).update(r)
    return {"power": phases, "device": torch.cuda.get_device_properties(dev).gcnArchName,
            "source": "amd-smi metric -p -c --json (socket_power, gfx_* clk)"}


def measure_peaks(fq, torch, dev, layers):
    """What this GPU reaches with the simplest kernels (include/flexq_peaks.h):
    a plain non-temporal read of each layer's packed-weight byte count and of 1 GiB
    (rotating over 3 buffers so no read is served from the MALL), and back-to-back
    int8 MFMAs with 0 and 8 independent FMAs per MFMA (8 = the fused rescale's count),
    with the shader clock of the MFMA loop, and the exact rescale's instruction mix
    without global memory (the rescale loop).  Medians of several launches."""
    sink = torch.empty(fq.peak_sink_bytes(), dtype=torch.uint8, device=dev)
    clock = torch.zeros(2, dtype=torch.int64, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        """Median event time of fn's launch.  A busy kernel (about 50 us) runs first
        each time, so the host has enqueued the start event, the launch and the end
        event before the GPU reaches them: the interval holds the kernel alone, not
        the host's launch latency."""
        fn()
        ts = []
        for _ in range(reps):
            fq.peak_mfma_i8(400, 0, sink, clock)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    out = {"hbm_read_gbs": {}}
    bufs = [torch.empty(1 << 30, dtype=torch.uint8, device=dev) for _ in range(3)]
    for b in bufs:
        b.fill_(1)
    sizes = {name: int(gemm_bytes(1, N, K)) // 16 * 16 for name, (N, K) in layers.items()}
    sizes["1GiB"] = 1 << 30
    for name, n in sizes.items():
        it = iter(range(1 << 30))
        ms = timed(lambda: fq.peak_hbm_read(bufs[next(it) % 3][:n], sink), 9)
        out["hbm_read_gbs"][name] = round(n / (ms * 1e-3) / 1e9, 1)
    del bufs
    for v, key in ((0, "mfma_i8"), (8, "mfma_i8_valu8")):
        iters = 4000
        ops = fq.peak_mfma_i8(iters, v, sink, clock)
        ms = timed(lambda: fq.peak_mfma_i8(iters, v, sink, clock), 5)
        c = clock.cpu().tolist()
        out[key + "_tops"] = round(ops / (ms * 1e-3) / 1e12, 1)
        out[key + "_clock_ghz"] = round(c[0] / c[1] * 0.1, 3)
    out["mfma_i8_valu8_frac_of_5pops"] = round(out["mfma_i8_valu8_tops"] / INT8_PEAK_TOPS, 4)
    # the exact rescale's own instruction mix (chained MFMAs, 4 fma + 4 DPP fmac per
    # MFMA, an LDS operand read per MFMA, a barrier per group): the ceiling of any
    # kernel that keeps the two FMAs per output and group
    iters = 2000
    ops = fq.peak_mfma_i8_rescale(iters, sink, clock)
    ms = timed(lambda: fq.peak_mfma_i8_rescale(iters, sink, clock), 5)
    c = clock.cpu().tolist()
    out["rescale_loop_tops"] = round(ops / (ms * 1e-3) / 1e12, 1)
    out["rescale_loop_clock_ghz"] = round(c[0] / c[1] * 0.1, 3)
    props = torch.cuda.get_device_properties(dev)
    out["device"] = getattr(props, "gcnArchName", props.name)
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(bufs, per_step, cols, packed, gpu_ms_per_step, tot_ops):
    """The oracle, as it is, on a bounded sample of the same step: for every distinct
    (M, abits, layer) of the step, the full activation quantization, and the GEMM
    restricted to its first `cols` output columns; the GEMM time is scaled linearly
    in N (exact: the work is linear in N) and each shape's time by the number of
    times a step runs it, to estimate the oracle's time for the whole step.  The GEMM
    runs on synth.default_threads() threads (the host cores this process may use,
    at most 16: the CPU share of one GPU on the benchmark's machines); two
    single-thread figures are added: the toy 16 x 256 x 512 layer and the 70B down
    projection at M = 1."""
    import oracle

    threads = synth.default_threads()
    q_time = 0.0
    g_time = 0.0
    g_time_scaled = 0.0
    wq = {}
    for name, (N, K) in LAYERS.items():
        wp, sw = packed[name][0]
        n = min(cols, N)
        wps = wp[: n * K * 3 // 16].cpu().numpy().view(np.uint32)  # first n/16 tiles
        sws = np.ascontiguousarray(sw[:, :n].cpu().numpy().T)      # [n][G] for the oracle
        wq[name] = (oracle.unpack_codes(wps, n, K), sws, n)
    q_time_step = 0.0
    for (M, ab, name), count in per_step.items():
        N, K = LAYERS[name]
        x = bufs[(M, name)][0]
        t = time.perf_counter()
        qa, sa = oracle.quant_act(x, ab)
        dq = time.perf_counter() - t
        q_time += dq
        q_time_step += dq * count
        qw, sws, n = wq[name]
        t = time.perf_counter()
        oracle.gemm(qa, sa, qw, sws, nthreads=threads)
        dt = time.perf_counter() - t
        g_time += dt
        g_time_scaled += dt * (N / n) * count
    est_step_s = q_time_step + g_time_scaled

    def single(M, N, K, seed):
        x = synth.activations(synth.derive_seed(seed, "x"), M, K)
        w = synth.weights(synth.derive_seed(seed, "w"), N, K)
        qa, sa = oracle.quant_act(x, 6)
        qw, sw = oracle.quant_w6(w)
        t = time.perf_counter()
        oracle.gemm(qa, sa, qw, sw, nthreads=1)
        return round(2.0 * M * N * K / (time.perf_counter() - t) / 1e9, 3)

    return {"value": round(tot_ops / est_step_s / 1e12, 5), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": (f"every distinct (M, abits, layer) of the step: full activation "
                       f"quantization ({q_time:.1f} s, 1 thread) and the GEMM on the first "
                       f"{cols} output columns ({g_time:.1f} s, {threads} threads), GEMM time "
                       f"scaled by N/{cols}; estimated oracle step {est_step_s:.0f} s vs GPU "
                       f"{gpu_ms_per_step:.2f} ms"),
            "sample_cpu_s": round(q_time + g_time, 1),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "single_thread_gops_toy_16x256x512": single(16, 256, 512, 7001),
            "single_thread_gops_70b_down_m1": single(1, 8192, 28672, 7002)}


if __name__ == "__main__":
    main()
