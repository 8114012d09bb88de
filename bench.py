"""Benchmark of the W6A6 / W6A8 linear-layer path on LLaMA-2-70B shapes, one MI355X.

A step is one pass of the hot path over one batch of synthetic input: for every
token count M in {1, 16, 64, 256, 1024, 4096}, both activation precisions (A6, A8)
and the four linear layers of a LLaMA-2-70B decoder block (qkv 10240x8192,
o 8192x8192, gate_up 57344x8192, down 8192x28672), quantize the fp16 activations
(flexq_quant_act) and run the W6Ax GEMM (flexq_gemm_w6ax) on packed 6-bit weights
resident in HBM.  Weights are packed once, before timing (offline step).

Prints one JSON line: value = whole-step GEMM+quant throughput in TOPS (2*M*N*K
integer ops per GEMM, M unpadded), per-shape TOPS / GB/s / roofline fractions,
the roofline of the dominant kernel and the CPU oracle timed on a bounded sample.
The step is first run launch by launch with events around every kernel (per-kernel
figures), then captured once as a HIP graph whose replays give ms_per_step and
value (the same kernels without host launch gaps; --eager keeps the eager time).
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


TILE_NAMES = {3: "256x128", 4: "128x128", 5: "128x64"}


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding over GPUs is designed, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import w6a6_w6a8_integer_amd as fq

    global LAYERS
    if args.layers == "70b_tp8":
        LAYERS = LAYERS_TP8
    fq.lib()
    dev = torch.device("cuda:0")
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

    # ---- weights: generated on the host, packed on the GPU, resident copies rotated
    # between launches so that no layer is served from the 256 MB MALL (at least two
    # copies and at least 1 GiB of packed weights in all)
    t0 = time.time()
    packed = {}
    set_bytes = sum(0.75 * N * K for N, K in LAYERS.values())
    ncopies = max(2, -(-(1 << 30) // int(set_bytes)))
    if (len(m_list) * len(ABITS) * len(LAYERS)) % ncopies == 0 and ncopies > 2:
        ncopies += 1  # a step's launch i then meets a different copy in every step
    if stack:
        ncopies = STACK_LAYERS  # one resident copy per decoder layer (same synthetic values)
    for li, (name, (N, K)) in enumerate(LAYERS.items()):
        w = synth.weights(synth.derive_seed(args.seed, "70b", name, "w"), N, K, nthreads=nthreads)
        wd = torch.from_numpy(w).to(dev)
        del w
        copies = []
        for c in range(ncopies):
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
            qa = torch.empty((M, K), dtype=torch.int8, device=dev)
            sa = torch.empty((K // GROUP, M), dtype=torch.float32, device=dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            bufs[(M, name)] = (x, xd, qa, sa, y)
    torch.cuda.synchronize()
    log(f"activations ready ({time.time() - t0:.1f} s)")

    # Largest M first: while the long prefill launches run, the host queues the rest of
    # the step, so the short decode launches at the end start back to back and their
    # events time the GPU, not the host's launch path.
    # Each launch: (M, abits, linear, weight copy or None = rotate through the copies).
    if stack:
        plan = [(M, 8 if layer in a8_layers else 6, name, layer)
                for M in sorted(m_list, reverse=True) for layer in range(STACK_LAYERS)
                for name in LAYERS]
    else:
        plan = [(M, ab, name, None) for M in sorted(m_list, reverse=True) for ab in ABITS
                for name in LAYERS]
    keys = sorted({e[:3] for e in plan}, key=lambda k: (-k[0], k[1], list(LAYERS).index(k[2])))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in plan]

    def step(timed: bool, s: int):
        for i, (M, ab, name, widx) in enumerate(plan):
            N, K = LAYERS[name]
            _, xd, qa, sa, y = bufs[(M, name)]
            wp, sw = packed[name][widx if widx is not None else (s * len(plan) + i) % ncopies]
            if timed:
                ev[i][0].record()
            fq.quant_act(xd, ab, q_a=qa, s_a=sa)
            if timed:
                ev[i][1].record()
            fq.gemm_w6ax(qa, sa, wp, sw, N, ab, y=y)
            if timed:
                ev[i][2].record()

    for s in range(args.warmup):
        step(False, s)
    torch.cuda.synchronize()

    quant_ms = {k: [] for k in keys}
    gemm_ms = {k: [] for k in keys}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_ms = []
    torch.cuda.synchronize()
    wall0 = time.time()
    start.record()
    for s in range(args.steps):
        step(True, s)
        torch.cuda.synchronize()  # read this step's events; the region stays back to back
        for i, e in enumerate(plan):
            quant_ms[e[:3]].append(ev[i][0].elapsed_time(ev[i][1]))
            gemm_ms[e[:3]].append(ev[i][1].elapsed_time(ev[i][2]))
        step_ms.append(ev[0][0].elapsed_time(ev[-1][2]))
    stop.record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    total_ms = start.elapsed_time(stop)
    ms_per_step_eager = statistics.median(step_ms)

    # The same step captured once as a HIP graph and replayed: the kernels and their
    # arguments are the eager step's (launch i reading weight copy i % ncopies), only
    # the host-side launch gaps between the kernels go.  Per-kernel figures above come
    # from the eager steps' events.
    graph_ms = None
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step(False, 0)
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

    # ---- aggregate
    shapes = []
    tot_ops = 0.0
    dec_ops = dec_bytes = dec_ms = 0.0
    pre_ops = pre_ms = 0.0
    for e in plan:
        tot_ops += 2.0 * e[0] * LAYERS[e[2]][0] * LAYERS[e[2]][1]
    for k in keys:
        M, ab, name = k
        N, K = LAYERS[name]
        g = statistics.median(gemm_ms[k])
        q = statistics.median(quant_ms[k])
        ops = 2.0 * M * N * K
        by = gemm_bytes(M, N, K)
        gsum = sum(gemm_ms[k])
        if fq.auto_path(M, N, K) == fq.PATH_DECODE:
            dec_ops += ops * len(gemm_ms[k])
            dec_bytes += by * len(gemm_ms[k])
            dec_ms += gsum
        else:
            pre_ops += ops * len(gemm_ms[k])
            pre_ms += gsum
        shapes.append({
            "layer": name, "M": M, "N": N, "K": K, "abits": ab,
            "kernel": "decode" if fq.auto_path(M, N, K) == fq.PATH_DECODE else "prefill",
            "tile": (None if fq.auto_path(M, N, K) == fq.PATH_DECODE else
                     TILE_NAMES[fq.prefill_tile(M, N, K)]),
            # columns a second prefill launch of 128 x 64 tiles covers (tail split)
            "tail_cols": (N - fq.prefill_main_cols(M, N, K)
                          if fq.auto_path(M, N, K) == fq.PATH_PREFILL else 0),
            "gemm_us": round(g * 1e3, 2), "quant_us": round(q * 1e3, 2),
            "tops": round(ops / (g * 1e-3) / 1e12, 2),
            "gbs": round(by / (g * 1e-3) / 1e9, 1),
            "frac_hbm": round(by / (g * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
            "frac_int8": round(ops / (g * 1e-3) / 1e12 / INT8_PEAK_TOPS, 3),
            "quant_gbs": round(quant_bytes(M, K) / (q * 1e-3) / 1e9, 1),
            "launches_per_step": len(gemm_ms[k]) // len(step_ms),
        })
    shapes.sort(key=lambda r: (r["M"], r["abits"], list(LAYERS).index(r["layer"])))
    ms_per_step = statistics.median(graph_ms) if graph_ms else ms_per_step_eager
    value = tot_ops / (ms_per_step * 1e-3) / 1e12

    pre_tops = pre_ops / (pre_ms * 1e-3) / 1e12 if pre_ms else 0.0
    # a prefill GEMM call is one kernel launch, two when the tail split applies
    pre_launches = sum(1 for (M, _, name, _) in plan
                       if fq.auto_path(M, *LAYERS[name]) == fq.PATH_PREFILL)
    pre_kernels = sum(1 + (fq.prefill_main_cols(M, *LAYERS[name]) < LAYERS[name][0])
                      for (M, _, name, _) in plan
                      if fq.auto_path(M, *LAYERS[name]) == fq.PATH_PREFILL)
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9 if dec_ms else 0.0
    if pre_ms >= dec_ms:
        # integer ops: the unit is TOP/s against the dense int8 MFMA peak
        roofline = {"kernel": "gemm_prefill_kernel", "bound": "mfma", "achieved": round(pre_tops, 1),
                    "peak": INT8_PEAK_TOPS, "unit": "TOP/s", "frac": round(pre_tops / INT8_PEAK_TOPS, 4),
                    # counters were taken on the default workload's launches only
                    "traffic": (recorded_traffic() if args.layers == "70b" and not args.m
                                else None),
                    "launches_per_step": pre_launches,
                    "kernel_launches_per_step": pre_kernels,
                    "ops_per_launch": round(pre_ops / len(step_ms) / max(pre_launches, 1))}
    else:
        roofline = {"kernel": "gemm_decode_kernel", "bound": "hbm", "achieved": round(dec_gbs, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                    "traffic": None}
    roofline_decode = {"kernel": "gemm_decode_kernel", "bound": "hbm", "achieved": round(dec_gbs, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(dec_gbs / HBM_PEAK_GBS, 4)}

    # the two target rows: HBM fraction over the M <= 16 GEMMs, int8 MFMA fraction over
    # the M >= 1024 GEMMs (algorithmic bytes / ops over summed event times)
    def frac_over(sel, num, peak, scale):
        ks = [k for k in keys if sel(k[0])]
        tot = sum(num(k) * len(gemm_ms[k]) for k in ks)
        ms = sum(sum(gemm_ms[k]) for k in ks)
        return round(tot / (ms * 1e-3) / scale / peak, 4) if ms else None
    targets = {
        "hbm_frac_m_le_16": frac_over(lambda M: M <= 16,
                                      lambda k: gemm_bytes(k[0], *LAYERS[k[2]]), HBM_PEAK_GBS, 1e9),
        "int8_frac_m_ge_1024": frac_over(lambda M: M >= 1024,
                                         lambda k: 2.0 * k[0] * LAYERS[k[2]][0] * LAYERS[k[2]][1],
                                         INT8_PEAK_TOPS, 1e12),
    }

    cpu = None
    if not args.no_cpu_baseline:
        per_step = {k: len(gemm_ms[k]) // len(step_ms) for k in keys}
        cpu = cpu_baseline(bufs, per_step, args.cpu_sample_cols, packed, ms_per_step, tot_ops)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "launch": "hip_graph" if graph_ms else "eager",
        "ms_per_step_eager": round(ms_per_step_eager, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.layers], "weight_copies": ncopies,
                   **({"stack_layers": STACK_LAYERS, "a8_layers": sorted(a8_layers)} if stack else {}),
                   "layers": {k: list(v) for k, v in LAYERS.items()}, "M": list(m_list),
                   "abits": list(ABITS), "group": GROUP, "step": "quant_act + gemm per (M, abits, layer)"},
        "roofline": roofline, "roofline_decode": roofline_decode, "targets": targets,
        "cpu_baseline": cpu,
        "timed_region_ms": round(total_ms, 2), "wall_s": round(wall, 2),
        "shapes": shapes,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(bufs, per_step, cols, packed, gpu_ms_per_step, tot_ops):
    """The oracle, as it is, on a bounded sample of the same step: for every distinct
    (M, abits, layer) of the step, the full activation quantization, and the GEMM
    restricted to its first `cols` output columns; the GEMM time is scaled linearly
    in N (exact: the work is linear in N) and each shape's time by the number of
    times a step runs it, to estimate the oracle's time for the whole step."""
    import oracle
    import torch

    threads = synth.default_threads()
    q_time = 0.0
    g_time = 0.0
    g_time_scaled = 0.0
    sample_ops = 0.0
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
        sample_ops += 2.0 * M * n * K
    est_step_s = q_time_step + g_time_scaled
    return {"value": round(tot_ops / est_step_s / 1e12, 5), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": (f"every distinct (M, abits, layer) of the step: full activation quantization "
                       f"({q_time:.1f} s, 1 thread) and the GEMM on the first {cols} output "
                       f"columns ({g_time:.1f} s, {threads} threads), GEMM time scaled by N/{cols}; "
                       f"estimated oracle step {est_step_s:.0f} s vs GPU {gpu_ms_per_step:.2f} ms"),
            "sample_cpu_s": round(q_time + g_time, 1)}


if __name__ == "__main__":
    main()
