"""Benchmark of the fused W4A16 path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--m 1]
                    [--workload llama8b_decode] [--no-prefill] [--no-cpu-baseline]

A step is one decode pass (M = 1 by default) over the four linears of a
Llama-3-8B-shaped decoder layer (qkv 6144x4096, o 4096x4096, gate_up
28672x4096, down 4096x14336), INT4 group-128 weights, BF16 activations.
Inputs are seeded synthetic tensors already resident in HBM; the packed
weights are replicated into enough distinct copies (>= 1 GiB) that every step
streams them from HBM rather than the 256 MB last-level cache.  Each copy's
four launches are captured in a HIP graph, and a rotation through all copies
in one more; the timed region replays K steps (whole rotations, then single
steps for any remainder) back to back between two device synchronisations.

value = algorithmic bytes per step / time per step, with algorithmic bytes
= packed codes + BF16 scales + INT32 zeros + X + Y.  Every figure is timed
after ~0.05-0.2 s of untimed runs of the same work (W = 4000 warm-up steps
for the headline): the GPU's clocks rise under sustained load, which the
vector work of the kernels feels (prefill most, 10-15%; decode a few %).

Also reported (same JSON line):
  roofline      the dominant kernel (the gate_up launch) timed alone with HIP
                events on its stream, against the 8 TB/s HBM peak;
  prefill       the same four layers at M = 4096 on the matrix-core kernel,
                TFLOP/s against the 2.5 PFLOP/s dense BF16 peak, timed after
                ~0.2 s of untimed GEMMs (the matrix cores' clocks rise under
                sustained load; every compute-bound figure is taken so);
  cpu_baseline  the CPU oracle on a bounded sample of the same step.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=4000)   # ~0.12 s of steps: steady clocks
    ap.add_argument("--m", type=int, default=1)
    ap.add_argument("--workload", default="llama8b_decode")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-m", type=int, default=4096)
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 40-layer decoder-stack stream (about 10.7 GB of packed weights)")
    ap.add_argument("--stack-tokens", type=int, default=30)
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the dense BF16 and naive-pipeline comparisons")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the decode sweep over the other M values and the 70B-shaped set")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the persistent chain decode (w4a16_chain_run)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(layer, M):
    N, K = layer.N, layer.K
    return N * K // 2 + (N * K // 128) * 6 + 2 * M * K + 2 * M * N


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec = gen.WORKLOADS[args.workload]
    layers = spec["layers"]
    M = args.m
    linear = w4.w4a16_gemv if M <= w4.GEMV_MAX_M else w4.w4a16_gemm

    # ---- inputs: pack each layer once, replicate packed copies past the LLC
    log(f"[bench] packing {args.workload} layers on {torch.cuda.get_device_name(0)}")
    packed, xs, ys = [], [], []
    for L in layers:
        W = gen.weights(L.N, L.K, args.workload, L.name, shift=spec["shift"], device=dev)
        packed.append(w4.w4a16_pack(W))
        del W
        xs.append(gen.activations(M, L.K, args.workload, L.name, device=dev))
        ys.append(torch.empty(M, L.N, dtype=torch.bfloat16, device=dev))
    set_bytes = sum(p.nbytes() for p in packed)
    ncopy = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    copies = [packed] + [[w4.PackedLinear(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                          for p in packed] for _ in range(ncopy - 1)]
    torch.cuda.synchronize()
    step_bytes = sum(decode_bytes(L, M) for L in layers)

    # ---- HIP graphs: one per copy (the four launches of one step) and one
    # for `rpg` whole rotations through the copies (ncopy steps in order,
    # ~40 steps per graph), so the host submits one graph per ~40 steps
    # instead of one per step (each graph launch costs some GPU time of its
    # own: ~1 us per step with one rotation of 10 steps per graph)
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for c in range(ncopy):  # warm the launch path before capture
            for p, x, y in zip(copies[c], xs, ys):
                linear(x, p, y)
        stream.synchronize()
        for c in range(ncopy):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for p, x, y in zip(copies[c], xs, ys):
                    linear(x, p, y)
            graphs.append(g)
        rpg = max(1, round(40 / ncopy))
        rotation = torch.cuda.CUDAGraph()
        with torch.cuda.graph(rotation, stream=stream):
            for _ in range(rpg):
                for c in range(ncopy):
                    for p, x, y in zip(copies[c], xs, ys):
                        linear(x, p, y)
    torch.cuda.synchronize()
    per_graph = rpg * ncopy

    def run_steps(n):
        """n decode steps, copy (s mod ncopy) at step s, as graphs of whole
        rotations plus single steps for the remainder."""
        for _ in range(n // per_graph):
            rotation.replay()
        for s in range(n - n % per_graph, n):
            graphs[s % ncopy].replay()

    with torch.cuda.stream(stream):
        run_steps(args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(args.steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] decode M={M}: {ms_per_step * 1e3:.2f} us/step, {value:.0f} GB/s over {ncopy} copies")

    # ---- dominant kernel alone: per-layer launch durations with HIP events
    def time_layer(i, reps=200):
        L = layers[i]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for r in range(reps):
                    linear(xs[i], copies[r % ncopy][i], ys[i])
        steady(stream, [g.replay], 0.05)
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        return us, decode_bytes(L, M) / (us * 1e-6) / 1e9

    per_layer = []
    for i, L in enumerate(layers):
        us, gbs = time_layer(i)
        per_layer.append({"layer": L.name, "N": L.N, "K": L.K, "us": round(us, 3),
                          "GBps": round(gbs, 1), "bytes": decode_bytes(L, M)})
        log(f"[bench]   {L.name:8s} N={L.N:6d} K={L.K:6d}: {us:8.2f} us {gbs:8.0f} GB/s")
    dom = max(range(len(layers)), key=lambda i: per_layer[i]["us"])
    roofline = {
        "bound": "hbm",
        "kernel": f"w4a16_gemv ({layers[dom].name}, N={layers[dom].N}, K={layers[dom].K}, M={M})",
        "achieved": per_layer[dom]["GBps"],
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(per_layer[dom]["GBps"] / HBM_PEAK_GBS, 4),
        "traffic": None,
    }
    del graphs
    torch.cuda.synchronize()

    # ---- a plain copy of known size: the reference that scales the HBM
    # byte counters of a profiling run (64 MiB read + 64 MiB written)
    cal_src = torch.zeros(16 << 20, dtype=torch.int32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            torch.add(cal_src, 1, out=cal_dst)
        stream.synchronize()
    del cal_src, cal_dst
    roofline["traffic"] = measured_traffic(layers[dom], M)

    # ---- the measured streaming-read ceiling (a plain read of 2 GiB, far
    # past the last-level cache) beside the specification's peak
    ceiling = hbm_read_ceiling(dev, stream)
    roofline["measured_ceiling_GBps"] = ceiling["GBps"]
    roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceiling["GBps"], 4)
    # the same read probe over exactly the dominant launch's bytes, one
    # launch per graph node over rotating buffers: what a plain stream of
    # that size reaches, launch cost included
    same = same_size_read(dev, stream, decode_bytes(layers[dom], M))
    ceiling["same_size_read"] = same
    roofline["same_size_read_us"] = same["us_per_launch"]
    roofline["frac_of_same_size_read"] = round(same["us_per_launch"] / per_layer[dom]["us"], 4)
    log(f"[bench] measured read ceiling: {ceiling['GBps']:.0f} GB/s "
        f"({ceiling['GBps'] / HBM_PEAK_GBS:.3f} of {HBM_PEAK_GBS:.0f})")

    # ---- the single 4096 x 4096 linear at M = 1 (same protocol)
    single = None
    if not args.no_sweep:
        single = single_linear(dev, stream)

    # ---- prefill GEMM on the same layers
    prefill = None
    if not args.no_prefill:
        Mp = args.prefill_m
        pxs = [gen.activations(Mp, L.K, "llama8b_prefill", L.name, device=dev) for L in layers]
        pys = [torch.empty(Mp, L.N, dtype=torch.bfloat16, device=dev) for L in layers]
        steady(stream, [lambda p=p, x=x, y=y: w4.w4a16_gemm(x, p, y) for p, x, y in zip(packed, pxs, pys)])
        with torch.cuda.stream(stream):
            reps = 10
            times = []
            for p, x, y in zip(packed, pxs, pys):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    w4.w4a16_gemm(x, p, y)
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1) * 1e-3 / reps)
        flops = [2.0 * Mp * L.N * L.K for L in layers]
        tf = sum(flops) / sum(times) / 1e12
        dom_p = max(range(len(layers)), key=lambda i: times[i])
        prefill = {
            "metric": f"prefill GEMM TFLOP/s (M={Mp})",
            "value": round(tf, 1), "unit": "TFLOP/s",
            "ms_per_step": round(sum(times) * 1e3, 4),
            "layers": [{"layer": L.name, "ms": round(t * 1e3, 4), "TFLOPs": round(f / t / 1e12, 1),
                        "split_k_workspace_bytes": gemm_split_bytes(Mp, L.N, L.K)}
                       for L, t, f in zip(layers, times, flops)],
            "roofline": {"bound": "mfma", "kernel": f"w4a16_gemm ({layers[dom_p].name}, M={Mp})",
                         "achieved": round(flops[dom_p] / times[dom_p] / 1e12, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops[dom_p] / times[dom_p] / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "traffic": None},
        }
        prefill["roofline"]["traffic"] = measured_traffic(
            layers[dom_p], Mp, "gemm_llama8b_prefill_m4096_traffic.json", ("gemm.hip", "common.h"))
        log(f"[bench] prefill M={Mp}: {tf:.1f} TFLOP/s")
        del pxs, pys
        # the other prefill batch sizes of the layer set, same protocol
        prefill["other_M"] = []
        for Mo in (512, 2048):
            if Mo == Mp:
                continue
            oxs = [gen.activations(Mo, L.K, "llama8b_prefill", L.name, device=dev) for L in layers]
            oys = [torch.empty(Mo, L.N, dtype=torch.bfloat16, device=dev) for L in layers]
            steady(stream, [lambda p=p, x=x, y=y: w4.w4a16_gemm(x, p, y) for p, x, y in zip(packed, oxs, oys)], 0.1)
            with torch.cuda.stream(stream):
                otimes = []
                for p, x, y in zip(packed, oxs, oys):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(reps):
                        w4.w4a16_gemm(x, p, y)
                    e1.record(stream)
                    e1.synchronize()
                    otimes.append(e0.elapsed_time(e1) * 1e-3 / reps)
            oflops = [2.0 * Mo * L.N * L.K for L in layers]
            otf = sum(oflops) / sum(otimes) / 1e12
            prefill["other_M"].append({
                "M": Mo, "TFLOPs": round(otf, 1), "ms_per_step": round(sum(otimes) * 1e3, 4),
                "layers": [{"layer": L.name, "ms": round(t * 1e3, 4), "TFLOPs": round(f / t / 1e12, 1),
                            "split_k_workspace_bytes": gemm_split_bytes(Mo, L.N, L.K)}
                           for L, t, f in zip(layers, otimes, oflops)]})
            log(f"[bench] prefill M={Mo}: {otf:.1f} TFLOP/s")
            del oxs, oys

    # ---- decode at the other batch sizes of the layer sets (same protocol)
    sweep = None
    if not args.no_sweep:
        sweep = [decode_sweep("llama8b_decode", [4, 8, 16, 32], dev, stream),
                 decode_sweep("llama70b_decode", [1, 8, 32], dev, stream)]

    # ---- the full decoder-stack weight stream: 40 layers x 4 linears, AWQ-
    # folded packing, one token = 160 dependent launches in one graph
    stack = None
    if not args.no_stack:
        stack = stack_decode(args.stack_tokens, dev, stream)

    # ---- the same layers as chains of dependent linears in one persistent
    # launch per token (w4a16_chain_run)
    chain = None
    if not args.no_chain:
        chain = {"llama8b_layer": chain_llama8b(dev, stream, steps=args.steps)}
        if not args.no_stack:
            chain["stack40"] = chain_stack(args.stack_tokens, dev, stream)

    # ---- the alternatives the fused path is chosen over (dense BF16 layers,
    # the naive expand-then-multiply pipeline)
    compare = None
    if not args.no_compare and args.workload == "llama8b_decode" and M == 1:
        compare = comparisons(args.workload, ms_per_step, prefill, dev, stream,
                              prefill_m=args.prefill_m)

    # ---- CPU oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, args.workload, spec, M, dev)
        if prefill is not None:
            cpu["prefill"] = cpu_baseline_prefill(layers, dev, args.prefill_m)
            prefill["cpu_baseline"] = cpu["prefill"]

    out = {
        "metric": "W4A16 decode GEMV achieved HBM GB/s (M=1) + prefill GEMM TFLOP/s (M=4096)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "bf16 activations x int4 weights (exact bf16 operands 128+q), fp32 accumulate, bf16 output",
        "data": "synthetic",
        "config": {"workload": workload_label(args.workload, spec),
                   "M": M, "step_bytes": step_bytes, "rotating_copies": ncopy, "steps_per_graph": per_graph,
                   "parallelism": "single GPU",
                   "headline_choice": "value is the decode step of the Llama-3-8B-shaped layer set at M=1, "
                                      "the configuration the metric is quoted on; the "
                                      "single 4096x4096 linear is under single_linear, the 70B-shaped set "
                                      "under decode_sweep and the 40-layer stack (the largest) under stack"},
        "per_layer": per_layer,
        "roofline": roofline,
        "prefill": prefill,
        "single_linear": single,
        "hbm_read_ceiling": ceiling,
        "decode_sweep": sweep,
        "stack": stack,
        "decode_chain": chain,
        "comparisons": compare,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def workload_label(name, spec):
    layers = ", ".join(f"{L.name} {L.N}x{L.K}" for L in spec["layers"])
    what = {"llama8b_decode": "Llama-3-8B-shaped decode layer set",
            "llama70b_decode": "70B-shaped decode layer set",
            "single_4096": "single linear",
            "llama8b_prefill": "Llama-3-8B-shaped layer set",
            "stack40_decode": "one layer of the 40-layer stack"}.get(name, name)
    return f"{name}: {what} ({layers}), INT4 group 128"


def hbm_read_ceiling(dev, stream, nbytes=2 << 30, reps=20):
    """Streaming-read rate of the library's plain read probe over a buffer of
    `nbytes` (far past the 256 MB last-level cache), HIP events on `stream`."""
    import torch
    import int4_weight_only_gemv_amd as w4
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            w4.w4a16_hbm_read_probe(buf, sink)
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            w4.w4a16_hbm_read_probe(buf, sink)
        e1.record(stream)
        e1.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del buf
    torch.cuda.synchronize()
    gbs = nbytes / sec / 1e9
    return {"GBps": round(gbs, 1), "bytes": nbytes, "reps": reps, "us_per_read": round(sec * 1e6, 2),
            "spec_GBps": HBM_PEAK_GBS, "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": "w4a16_hbm_read_probe (16-byte loads, 1 KiB per wave instruction)"}


def same_size_read(dev, stream, nbytes, reps=200):
    """The read probe over `nbytes` (rounded down to 16 bytes) per launch,
    a graph of `reps` launches over rotating buffers (>= 1 GiB in all),
    timed with HIP events on `stream`."""
    import torch
    import int4_weight_only_gemv_amd as w4
    n16 = nbytes // 16
    ncopy = max(2, math.ceil(ROTATE_BYTES / (16 * n16)))
    bufs = [torch.ones(4 * n16, dtype=torch.int32, device=dev) for _ in range(ncopy)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    us = _graph_us(stream, lambda r: w4.w4a16_hbm_read_probe(bufs[r % ncopy], sink), reps)
    del bufs
    torch.cuda.synchronize()
    return {"bytes": 16 * n16, "us_per_launch": round(us, 3), "GBps": round(16 * n16 / (us * 1e-6) / 1e9, 1),
            "rotating_buffers": ncopy, "launches_timed": reps}


def single_linear(dev, stream, M=1, reps=400):
    """The single 4096 x 4096 linear (the first config) at M = 1: one launch
    per replay over rotating packed copies (>= 1 GiB), a graph of `reps`
    launches timed with HIP events on `stream`."""
    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen
    spec = gen.WORKLOADS["single_4096"]
    L = spec["layers"][0]
    W = gen.weights(L.N, L.K, "single_4096", L.name, device=dev)
    p = w4.w4a16_pack(W)
    del W
    ncopy = max(2, math.ceil(ROTATE_BYTES / p.nbytes()))
    copies = [p] + [w4.PackedLinear(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                    for _ in range(ncopy - 1)]
    x = gen.activations(M, L.K, "single_4096", L.name, device=dev)
    y = torch.empty(M, L.N, dtype=torch.bfloat16, device=dev)
    us = _graph_us(stream, lambda r: w4.w4a16_gemv(x, copies[r % ncopy], y), reps)
    nbytes = decode_bytes(L, M)
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] single 4096x4096 M={M}: {us:.2f} us, {gbs:.0f} GB/s")
    del copies
    torch.cuda.synchronize()
    return {"workload": workload_label("single_4096", spec), "M": M, "bytes": nbytes,
            "us_per_launch": round(us, 3), "GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "rotating_copies": ncopy,
            "launches_timed": reps}


def gemm_split_bytes(M, N, K) -> int:
    """The workspace with which w4a16_gemm splits K for this shape (0: the
    shape runs unsplit)."""
    import ctypes
    import int4_weight_only_gemv_amd as w4
    n = ctypes.c_int64(0)
    w4._check("w4a16_gemm_workspace_bytes", w4.lib.w4a16_gemm_workspace_bytes(M, N, K, ctypes.byref(n)))
    return int(n.value)


def kernel_source_digest(files=("gemv.hip", "common.h")) -> str:
    """sha256 of a kernel's sources (the counters recorded under profiles/
    only apply to the code they were taken on)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "int4_weight_only_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(layer, M, name="gemv_llama8b_decode_m1_traffic.json",
                     sources=("gemv.hip", "common.h")):
    """HBM bytes per launch of a dominant launch, from the FETCH_SIZE and
    WRITE_SIZE counters recorded in profiles/ (each scaled by what the
    counter read for a copy of known size), or None when they were taken on
    other kernel sources or another shape."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha256") != kernel_source_digest(sources):
        return None
    if (rec.get("N"), rec.get("K"), rec.get("M")) != (layer.N, layer.K, M):
        return None
    return rec.get("hbm_bytes_per_launch")


def decode_sweep(workload, Ms, dev, stream, steps=40, replays=5):
    """Decode throughput of one layer set at several batch sizes M: the four
    launches of a step in order, replicated weight copies past the last-level
    cache, a graph of `steps` steps replayed for ~0.1 s untimed, then
    `replays` times timed with HIP events on its stream."""
    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen
    spec = gen.WORKLOADS[workload]
    layers = spec["layers"]
    packed = []
    for L in layers:
        W = gen.weights(L.N, L.K, workload, L.name, shift=spec["shift"], device=dev)
        packed.append(w4.w4a16_pack(W))
        del W
    set_bytes = sum(p.nbytes() for p in packed)
    ncopy = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    copies = [packed] + [[w4.PackedLinear(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                          for p in packed] for _ in range(ncopy - 1)]
    rows = []
    for M in Ms:
        xs = [gen.activations(M, L.K, workload, L.name, device=dev) for L in layers]
        ys = [torch.empty(M, L.N, dtype=torch.bfloat16, device=dev) for L in layers]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for p, x, y in zip(packed, xs, ys):
                w4.w4a16_gemv(x, p, y)
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for s in range(steps):
                    for p, x, y in zip(copies[s % ncopy], xs, ys):
                        w4.w4a16_gemv(x, p, y)
        # the matrix-core and dot-product kernels at these M do more vector
        # work per byte than M = 1: warm the clocks as for prefill
        steady(stream, [g.replay], 0.1)
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(replays):
                g.replay()
            e1.record(stream)
            e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (steps * replays)
        nbytes = sum(decode_bytes(L, M) for L in layers)
        gbs = nbytes / (us * 1e-6) / 1e9
        rows.append({"M": M, "us_per_step": round(us, 3), "GBps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        log(f"[bench] {workload} M={M}: {us:.2f} us/step, {gbs:.0f} GB/s")
        del g, xs, ys
    del copies, packed
    torch.cuda.synchronize()
    return {"workload": workload, "step_bytes_M1": sum(decode_bytes(L, 1) for L in layers),
            "rotating_copies": ncopy, "steps_per_graph": steps, "graph_replays_timed": replays,
            "results": rows}


def _graph_us(stream, body, reps):
    """Average microseconds of `body` over `reps` replays captured in one
    graph (after ~0.05 s of untimed replays), timed with HIP events on
    `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        body(0)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for r in range(reps):
                body(r)
    steady(stream, [g.replay], 0.05)
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def steady(stream, calls, seconds=0.2):
    """Run `calls` round-robin on `stream` for about `seconds` of GPU time
    (untimed).  The matrix cores' clocks rise under sustained load: the
    first ~100 ms of back-to-back GEMMs run up to 15% slower than the
    steady state, so every compute-bound figure is taken after this."""
    import torch
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        while True:
            for c in calls:
                c()
            stream.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break


def comparisons(workload, fused_ms_per_step, fused_prefill, dev, stream, steps=40, prefill_m=4096):
    """The alternatives the fused path is chosen over, on the same layer set
    and step protocol (weights past the last-level cache, graphs of whole
    steps):
      dense BF16 decode (M=1): the dense layer the INT4 weights replace, and
        the decode cost of an offline BF16 expansion of them;
      naive three-kernel decode: expand each layer's packed weights to a BF16
        buffer, then the dense product (an HBM round trip per layer);
      dense BF16 prefill (M=prefill_m) on this library's matrix-core kernel,
        and torch's BF16 linear (hipBLASLt) for context."""
    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen
    spec = gen.WORKLOADS[workload]
    layers = spec["layers"]
    out = {}
    # dense BF16 weights: the generator's weights, the model before quantising
    dense = [gen.weights(L.N, L.K, workload, L.name, shift=spec["shift"], device=dev) for L in layers]
    dense_bytes = sum(w.numel() * 2 for w in dense)
    ncopy = max(2, math.ceil(ROTATE_BYTES / dense_bytes))
    dcopies = [dense] + [[w.clone() for w in dense] for _ in range(ncopy - 1)]
    xs = [gen.activations(1, L.K, workload, L.name, device=dev) for L in layers]
    ys = [torch.empty(1, L.N, dtype=torch.bfloat16, device=dev) for L in layers]

    def dense_step(s):
        for w, x, y in zip(dcopies[s % ncopy], xs, ys):
            w4.w4a16_dense_gemv(x, w, y)
    us_dense = _graph_us(stream, dense_step, steps)
    step_dense_bytes = dense_bytes + sum(2 * (L.K + L.N) for L in layers)
    del dcopies
    torch.cuda.synchronize()

    packed = [w4.w4a16_pack(w) for w in dense]
    pset = sum(p.nbytes() for p in packed)
    pcopy = max(2, math.ceil(ROTATE_BYTES / pset))
    pcopies = [packed] + [[w4.PackedLinear(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                           for p in packed] for _ in range(pcopy - 1)]
    scratch = [torch.empty(L.N, L.K, dtype=torch.bfloat16, device=dev) for L in layers]

    def naive_step(s):
        for p, buf, x, y in zip(pcopies[s % pcopy], scratch, xs, ys):
            w4.w4a16_dequantize_bf16(p, out=buf)
            w4.w4a16_dense_gemv(x, buf, y)
    us_naive = _graph_us(stream, naive_step, steps)

    def expand_only(s):
        for p, buf in zip(pcopies[s % pcopy], scratch):
            w4.w4a16_dequantize_bf16(p, out=buf)
    us_expand = _graph_us(stream, expand_only, steps)
    fused_us = fused_ms_per_step * 1e3
    out["decode_M1"] = {
        "fused_w4a16_us_per_step": round(fused_us, 3),
        "dense_bf16_us_per_step": round(us_dense, 3),
        "dense_bf16_GBps": round(step_dense_bytes / (us_dense * 1e-6) / 1e9, 1),
        "speedup_fused_vs_dense": round(us_dense / fused_us, 3),
        "offline_expansion_decode_us_per_step": round(us_dense, 3),
        "naive_three_kernel_us_per_step": round(us_naive, 3),
        "naive_expand_kernels_us_per_step": round(us_expand, 3),
        "speedup_fused_vs_naive": round(us_naive / fused_us, 3),
        "dense_rotating_copies": ncopy,
    }
    log(f"[bench] compare decode M=1: fused {fused_us:.1f} us, dense bf16 {us_dense:.1f} us "
        f"({us_dense / fused_us:.2f}x), naive 3-kernel {us_naive:.1f} us ({us_naive / fused_us:.2f}x)")
    del pcopies, scratch, xs, ys
    torch.cuda.synchronize()

    # prefill: dense BF16 on this library's matrix-core kernel and torch's
    if fused_prefill is not None:
        Mp = prefill_m
        pxs = [gen.activations(Mp, L.K, "llama8b_prefill", L.name, device=dev) for L in layers]
        pys = [torch.empty(Mp, L.N, dtype=torch.bfloat16, device=dev) for L in layers]
        t_dense, t_torch = [], []
        for w, x, y in zip(dense, pxs, pys):
            steady(stream, [lambda w=w, x=x, y=y: w4.w4a16_dense_gemm(x, w, y)], 0.1)
            t_dense.append(_graph_us(stream, lambda r, w=w, x=x, y=y: w4.w4a16_dense_gemm(x, w, y), 5))
            # torch's BF16 product, eager, on a contiguous K x N copy (no
            # transposed operand views, no graph capture of library calls)
            wt = w.t().contiguous()
            steady(stream, [lambda x=x, wt=wt, y=y: torch.mm(x, wt, out=y)], 0.1)
            with torch.cuda.stream(stream):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    torch.mm(x, wt, out=y)
                e1.record(stream)
                e1.synchronize()
            t_torch.append(e0.elapsed_time(e1) * 1e3 / 5)
            del wt
        flops = sum(2.0 * Mp * L.N * L.K for L in layers)
        tf_dense = flops / (sum(t_dense) * 1e-6) / 1e12
        tf_torch = flops / (sum(t_torch) * 1e-6) / 1e12
        out[f"prefill_M{Mp}"] = {
            "fused_w4a16_TFLOPs": fused_prefill["value"],
            "dense_bf16_TFLOPs": round(tf_dense, 1),
            "ratio_fused_vs_dense": round(fused_prefill["value"] / tf_dense, 3),
            "torch_bf16_linear_TFLOPs": round(tf_torch, 1),
            "layers": [{"layer": L.name, "dense_ms": round(a * 1e-3, 4), "torch_ms": round(b * 1e-3, 4)}
                       for L, a, b in zip(layers, t_dense, t_torch)],
        }
        log(f"[bench] compare prefill M={Mp}: fused {fused_prefill['value']:.1f}, dense bf16 "
            f"{tf_dense:.1f}, torch bf16 {tf_torch:.1f} TFLOP/s")
        del pxs, pys
    # output error of the quantised layer against the dense BF16 layer,
    # asymmetric (the format) and symmetric (the variant the pages argue
    # wastes range), on plain weights and on weights with per-group offsets
    errs = []
    Mq = 64
    for shift in (False, True):
        for L in layers:
            W = gen.weights(L.N, L.K, workload, L.name, shift=shift, device=dev)
            X = gen.activations(Mq, L.K, workload, L.name, device=dev)
            yd = w4.w4a16_dense_gemm(X, W).float()
            row = {"layer": L.name, "group_offsets": shift}
            for name, pk in (("asymmetric", w4.w4a16_pack), ("symmetric", w4.w4a16_pack_symmetric)):
                yq = w4.w4a16_gemm(X, pk(W)).float()
                row[f"{name}_rel_l2"] = round(float((yq - yd).norm() / yd.norm()), 5)
            errs.append(row)
            del W, X, yd, yq
    out["quantisation_error_vs_dense"] = {"M": Mq, "layers": errs}

    # W8A16 decode step (M=1), same protocol: the pages' precision matrix puts
    # its decode gain over 16-bit weights at about 1.5x
    i8 = [w4.w4a16_pack_int8(w) for w in dense]
    iset = sum(p.nbytes() for p in i8)
    icopy = max(2, math.ceil(ROTATE_BYTES / iset))
    icopies = [i8] + [[w4.PackedLinearInt8(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                       for p in i8] for _ in range(icopy - 1)]
    ixs = [gen.activations(1, L.K, workload, L.name, device=dev) for L in layers]
    iys = [torch.empty(1, L.N, dtype=torch.bfloat16, device=dev) for L in layers]

    def int8_step(s):
        for p, x, y in zip(icopies[s % icopy], ixs, iys):
            w4.w4a16_gemv_int8(x, p, y)
    us_i8 = _graph_us(stream, int8_step, steps)
    i8_bytes = iset + sum(2 * (L.K + L.N) for L in layers)
    rel8 = []
    for L, W, p in zip(layers, dense, i8):
        X = gen.activations(1, L.K, workload, L.name, device=dev)
        yd = w4.w4a16_dense_gemv(X, W).float()
        y8 = w4.w4a16_gemv_int8(X, p).float()
        rel8.append(round(float((y8 - yd).norm() / yd.norm()), 6))
    out["w8a16_decode_M1"] = {
        "us_per_step": round(us_i8, 3), "GBps": round(i8_bytes / (us_i8 * 1e-6) / 1e9, 1),
        "speedup_vs_dense_bf16": round(us_dense / us_i8, 3),
        "w4a16_speedup_vs_w8a16": round(us_i8 / fused_us, 3),
        "rotating_copies": icopy, "rel_l2_vs_dense": rel8,
    }
    if fused_prefill is not None:
        t8 = []
        for L, p in zip(layers, i8):
            x = gen.activations(prefill_m, L.K, "llama8b_prefill", L.name, device=dev)
            y = torch.empty(prefill_m, L.N, dtype=torch.bfloat16, device=dev)
            steady(stream, [lambda x=x, p=p, y=y: w4.w4a16_gemm_int8(x, p, y)], 0.1)
            t8.append(_graph_us(stream, lambda r, x=x, p=p, y=y: w4.w4a16_gemm_int8(x, p, y), 5))
            del x, y
        flops = sum(2.0 * prefill_m * L.N * L.K for L in layers)
        out[f"w8a16_prefill_M{prefill_m}"] = {
            "TFLOPs": round(flops / (sum(t8) * 1e-6) / 1e12, 1),
            "layers_ms": [round(t * 1e-3, 4) for t in t8]}
        log(f"[bench] W8A16 prefill M={prefill_m}: {flops / (sum(t8) * 1e-6) / 1e12:.1f} TFLOP/s")
    log(f"[bench] W8A16 decode M=1: {us_i8:.1f} us/step ({i8_bytes / (us_i8 * 1e-6) / 1e9:.0f} GB/s), "
        f"{us_dense / us_i8:.2f}x dense bf16; rel l2 {max(rel8):.5f}")
    del icopies, ixs, iys, i8
    torch.cuda.synchronize()

    # quantisation groups of 32 / 64 / 128 inputs: decode step (M=1, same
    # protocol as the headline), prefill at prefill_m, and the output error
    # against the dense BF16 layer
    groups = []
    for group in (32, 64, 128):
        gpk = [w4.w4a16_pack(w, group=group) for w in dense]
        gset = sum(p.nbytes() for p in gpk)
        gcopy = max(2, math.ceil(ROTATE_BYTES / gset))
        gcopies = [gpk] + [[w4.PackedLinear(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                            for p in gpk] for _ in range(gcopy - 1)]
        gxs = [gen.activations(1, L.K, workload, L.name, device=dev) for L in layers]
        gys = [torch.empty(1, L.N, dtype=torch.bfloat16, device=dev) for L in layers]

        def group_step(s, gcopies=gcopies, gxs=gxs, gys=gys):
            for p, x, y in zip(gcopies[s % len(gcopies)], gxs, gys):
                w4.w4a16_gemv(x, p, y)
        us = _graph_us(stream, group_step, steps)
        step_bytes = gset + sum(2 * (L.K + L.N) for L in layers)
        row = {"group": group, "bits_per_weight": round(8.0 * gset / sum(L.N * L.K for L in layers), 3),
               "decode_M1_us_per_step": round(us, 3),
               "decode_M1_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1)}
        del gcopies, gxs, gys
        torch.cuda.synchronize()
        if fused_prefill is not None:
            t = []
            for L, p in zip(layers, gpk):
                x = gen.activations(prefill_m, L.K, "llama8b_prefill", L.name, device=dev)
                y = torch.empty(prefill_m, L.N, dtype=torch.bfloat16, device=dev)
                steady(stream, [lambda x=x, p=p, y=y: w4.w4a16_gemm(x, p, y)], 0.1)
                t.append(_graph_us(stream, lambda r, x=x, p=p, y=y: w4.w4a16_gemm(x, p, y), 5))
                del x, y
            flops = sum(2.0 * prefill_m * L.N * L.K for L in layers)
            row[f"prefill_M{prefill_m}_TFLOPs"] = round(flops / (sum(t) * 1e-6) / 1e12, 1)
        rel = []
        for L, W, p in zip(layers, dense, gpk):
            X = gen.activations(64, L.K, workload, L.name, device=dev)
            yd = w4.w4a16_dense_gemm(X, W).float()
            yq = w4.w4a16_gemm(X, p).float()
            rel.append(float((yq - yd).norm() / yd.norm()))
        row["rel_l2_vs_dense"] = [round(v, 5) for v in rel]
        groups.append(row)
        log(f"[bench] group {group}: decode {row['decode_M1_us_per_step']:.1f} us/step "
            f"({row['decode_M1_GBps']:.0f} GB/s), prefill {row.get(f'prefill_M{prefill_m}_TFLOPs')} "
            f"TFLOP/s, rel l2 {max(rel):.4f}")
        del gpk
        torch.cuda.synchronize()
    out["group_sizes"] = groups

    # AWQ exponent search on the library's kernels: calibration tokens from
    # one batch, the error measured on another; the recipe's weights (their
    # salient input channels already x8) and, as a contrast, the same layers
    # with those weight columns at ordinary size
    alphas = [round(0.1 * i, 1) for i in range(11)]
    search = []
    for contrast in (False, True):
        for L in layers:
            W = gen.weights(L.N, L.K, workload, L.name, device=dev)
            if contrast:
                S = gen.salient_channels(L.K, workload, L.name).to(dev)
                W[:, S] = (W[:, S].float() / 8.0).to(torch.bfloat16)
            Xc = gen.activations(512, L.K, workload, L.name, role="Xcal", device=dev)
            Xe = gen.activations(256, L.K, workload, L.name, role="Xeval", device=dev)
            best, e = w4.w4a16_awq_search(W, Xc, alphas, Xe)
            search.append({"layer": L.name, "salient_weights_x8": not contrast, "best_alpha": alphas[best],
                           "error_alpha0": round(e[0], 5), "error_best": round(e[best], 5),
                           "errors": [round(v, 5) for v in e]})
            del W, Xc, Xe
    out["awq_search"] = {"alphas": alphas, "calibration_tokens": 512, "eval_tokens": 256,
                         "layers": search}
    log("[bench] AWQ search: " + ", ".join(
        f"{r['layer']}{'' if r['salient_weights_x8'] else '(w1)'} a={r['best_alpha']} "
        f"{r['error_alpha0']:.4f}->{r['error_best']:.4f}" for r in search))
    log("[bench] compare error vs dense: " + ", ".join(
        f"{r['layer']}{'+off' if r['group_offsets'] else ''} asym {r['asymmetric_rel_l2']:.4f} "
        f"sym {r['symmetric_rel_l2']:.4f}" for r in errs))
    del dense, packed
    torch.cuda.synchronize()
    return out


def stack_decode(tokens, dev, stream, Ms=(1, 8)):
    """Decode of a 40-layer stack (hidden 5120, 40 q / 8 kv heads of 128,
    SwiGLU 27648): each layer's four linears packed from their own seeded
    weights after an AWQ pre-scale s = importance^0.5 from a synthetic
    512-token calibration batch; activations X' = X * (1/s) as the folded
    producer would emit them.  One token runs the 160 linears in order, at
    each M in Ms (GEMV); the stack (~10.7 GB) is far larger than the
    last-level cache, so every token streams it from HBM."""
    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen
    spec = gen.WORKLOADS["stack40_decode"]
    cfg, layers, depth = "stack40_decode", spec["layers"], spec["depth"]
    t0 = time.perf_counter()
    seq = []   # (packed, gamma', layer, name) per linear, in execution order
    for d in range(depth):
        for L in layers:
            name = f"{L.name}.{d}"
            W = gen.weights(L.N, L.K, cfg, name, device=dev)
            xcal = gen.activations(spec["calib_tokens"], L.K, cfg, name, role="Xcal", device=dev)
            s_awq = w4.w4a16_awq_scale(w4.w4a16_awq_importance(xcal), spec["awq_alpha"])
            p = w4.w4a16_pack(W, awq_s=s_awq)
            gamma = torch.ones(L.K, dtype=torch.bfloat16, device=dev)
            w4.w4a16_awq_fold(s_awq, gamma)
            seq.append((p, gamma, L, name))
            del W, xcal
    torch.cuda.synchronize()
    log(f"[bench] stack: {len(seq)} linears, "
        f"{sum(decode_bytes(L, 1) for L in layers) * depth / 1e9:.2f} GB per token, "
        f"built in {time.perf_counter() - t0:.1f} s")
    results = []
    for M in Ms:
        run = [(p, w4.w4a16_scale_channels(gen.activations(M, L.K, cfg, name, device=dev), gamma),
                torch.empty(M, L.N, dtype=torch.bfloat16, device=dev)) for p, gamma, L, name in seq]
        nbytes = sum(decode_bytes(L, M) for L in layers) * depth
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for p, x, y in run:
                w4.w4a16_gemv(x, p, y)
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for p, x, y in run:
                    w4.w4a16_gemv(x, p, y)
        steady(stream, [g.replay], 0.1)
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(tokens):
                g.replay()
            e1.record(stream)
            e1.synchronize()
        ms = e0.elapsed_time(e1) / tokens
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"[bench] stack decode M={M}: {ms:.3f} ms/token, {gbs:.0f} GB/s")
        results.append({"M": M, "bytes_per_token": nbytes, "ms_per_token": round(ms, 4),
                        "tokens_per_s": round(M * 1e3 / ms, 1), "GBps": round(gbs, 1),
                        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        del run, g
    del seq
    torch.cuda.synchronize()
    return {"workload": "40-layer decoder stack (hidden 5120, 40/8 heads of 128, SwiGLU 27648), "
                        "INT4 group 128, AWQ alpha 0.5", "linears_per_token": 4 * depth,
            "tokens_timed": tokens, "results": results}


def host_threads() -> int:
    return len(os.sched_getaffinity(0))


LLAMA8B_CHAIN = [("qkv", "x0", None), ("o", "attn1", (5120, 128, 4)), ("gate_up", "prev", None),
                 ("down", "swiglu", None)]


def chain_llama8b(dev, stream, steps=200, Ms=(1, 2)):
    """The Llama-3-8B-shaped layer set as a decoder layer: qkv -> attention
    over a one-token context -> o -> gate_up -> SwiGLU -> down, each linear's
    input formed from the previous output, one persistent launch per token
    (w4a16_chain_run), over rotating weight copies (>= 1 GiB) so that every
    token streams its weights from HBM; HIP events on `stream`."""
    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen
    spec = gen.WORKLOADS["llama8b_decode"]
    layers = spec["layers"]
    packed = []
    for L in layers:
        W = gen.weights(L.N, L.K, "llama8b_decode", L.name, device=dev)
        packed.append(w4.w4a16_pack(W))
        del W
    set_bytes = sum(p.nbytes() for p in packed)
    ncopy = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    copies = [packed] + [[w4.PackedLinear(p.codes.clone(), p.scales.clone(), p.zeros.clone())
                          for p in packed] for _ in range(ncopy - 1)]
    rows = []
    for M in Ms:
        outs = None
        plans = []
        for c in range(ncopy):
            lin = [dict(p=p, input=kind, params=params) for p, (_, kind, params) in zip(copies[c], LLAMA8B_CHAIN)]
            pl = w4.w4a16_chain_prepare(lin, M, outputs=outs)
            outs = pl.outputs
            plans.append(pl)
        x0 = gen.activations(M, layers[0].K, "llama8b_decode", "chain_x0", device=dev)
        steady(stream, [lambda pl=pl: w4.w4a16_chain_run(pl, x0) for pl in plans], 0.1)
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for s_ in range(steps):
                w4.w4a16_chain_run(plans[s_ % ncopy], x0)
            e1.record(stream)
            e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        assert w4.w4a16_chain_status(plans[0]) == 0, "chain barrier timeout"
        nbytes = sum(decode_bytes(L, M) for L in layers)
        gbs = nbytes / (us * 1e-6) / 1e9
        rows.append({"M": M, "us_per_step": round(us, 3), "GBps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "step_bytes": nbytes})
        log(f"[bench] chain llama8b layer M={M}: {us:.2f} us/step, {gbs:.0f} GB/s")
        del plans
    del copies, packed
    torch.cuda.synchronize()
    return {"workload": "llama8b_decode as one decoder layer: qkv -> attention over one token -> o -> gate_up "
                        "-> SwiGLU -> down (INT4 group 128), one persistent launch per token",
            "rotating_copies": ncopy, "steps": steps, "results": rows}


def chain_stack(tokens, dev, stream, Ms=(1, 2)):
    """The 40-layer stack as one chain of 160 dependent linears (qkv <- down
    of the layer before, o <- attention over one token, gate_up <- o, down
    <- SwiGLU), AWQ-folded packing with each linear's producer weight
    gamma' = bf16(1/s) applied as its input is formed; one persistent launch
    per token (~10.7 GB of weights, far past the last-level cache)."""
    import torch
    import int4_weight_only_gemv_amd as w4
    from synth import gen
    spec = gen.WORKLOADS["stack40_decode"]
    cfg, layers, depth = "stack40_decode", spec["layers"], spec["depth"]
    kinds = {"qkv": ("prev", None), "o": ("attn1", (5120 + 1024, 128, 5)), "gate_up": ("prev", None),
             "down": ("swiglu", None)}
    lin = []
    for d in range(depth):
        for L in layers:
            name = f"{L.name}.{d}"
            W = gen.weights(L.N, L.K, cfg, name, device=dev)
            xcal = gen.activations(spec["calib_tokens"], L.K, cfg, name, role="Xcal", device=dev)
            s_awq = w4.w4a16_awq_scale(w4.w4a16_awq_importance(xcal), spec["awq_alpha"])
            p = w4.w4a16_pack(W, awq_s=s_awq)
            gamma = torch.ones(L.K, dtype=torch.bfloat16, device=dev)
            w4.w4a16_awq_fold(s_awq, gamma)
            kind, params = kinds[L.name]
            if d == 0 and L.name == "qkv":
                kind = "x0"
            lin.append(dict(p=p, input=kind, params=params, gamma=gamma))
            del W, xcal
    torch.cuda.synchronize()
    rows = []
    for M in Ms:
        plan = w4.w4a16_chain_prepare(lin, M)
        x0 = gen.activations(M, layers[0].K, cfg, "chain_x0", device=dev)
        steady(stream, [lambda: w4.w4a16_chain_run(plan, x0)], 0.1)
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(tokens):
                w4.w4a16_chain_run(plan, x0)
            e1.record(stream)
            e1.synchronize()
        ms = e0.elapsed_time(e1) / tokens
        assert w4.w4a16_chain_status(plan) == 0, "chain barrier timeout"
        nbytes = sum(decode_bytes(L, M) for L in layers) * depth
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"[bench] chain stack M={M}: {ms:.3f} ms/token, {gbs:.0f} GB/s")
        rows.append({"M": M, "bytes_per_token": nbytes, "ms_per_token": round(ms, 4),
                     "tokens_per_s": round(M * 1e3 / ms, 1), "GBps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        del plan
    del lin
    torch.cuda.synchronize()
    return {"workload": "40-layer decoder stack (hidden 5120, 40/8 heads of 128, SwiGLU 27648) as one chain of "
                        "160 dependent linears, INT4 group 128, AWQ alpha 0.5 folded into each producer weight",
            "tokens_timed": tokens, "results": rows}


def cpu_baseline(layers, workload, spec, M, dev, row_stride=2, min_seconds=10.0):
    """Time the CPU oracle (unpack, dequantise, fp64 dot) for the same step on
    every `row_stride`-th output row of each layer, with the BLAS thread pool
    at the host's core count (the unpack and dequantise steps are numpy
    elementwise operations on one thread)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    from synth import gen

    prepared = []
    for L in layers:
        W = gen.weights(L.N, L.K, workload, L.name, shift=spec["shift"], device=dev)
        rows = torch.arange(0, L.N, row_stride, device=dev)
        Wb = gen.bits(W[rows])
        del W
        X = gen.bits(gen.activations(M, L.K, workload, L.name, device=dev))
        codes, scales, zeros = O.quantize_pack(Wb)   # untimed: the oracle's own packing
        prepared.append((L, X, codes, scales, zeros, len(rows)))
    nbytes = 0
    t0 = time.perf_counter()
    reps = 0
    cores = host_threads()
    with threadpool_limits(limits=cores):
        while True:
            for L, X, codes, scales, zeros, nr in prepared:
                O.matmul_ref(X, codes, scales, zeros)
                nbytes += nr * L.K // 2 + nr * (L.K // 128) * 6 + 2 * M * L.K + 2 * M * nr
            reps += 1
            if time.perf_counter() - t0 >= min_seconds or reps >= 50:
                break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"one output row in {row_stride} of each of the four layers, M={M}, "
                      f"{reps} pass(es); unpack + dequantise + fp64 dot (BLAS on {cores} threads)"}


def cpu_baseline_prefill(layers, dev, M, rows=128, xrows=512, min_seconds=10.0):
    """The CPU oracle on a bounded sample of the prefill step: `rows` output
    rows of each layer against a seeded sample of `xrows` of the M activation
    rows, timed and scaled to TFLOP/s of the sample's own work."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    from synth import gen
    prepared = []
    rng = np.random.default_rng(4096)
    for L in layers:
        W = gen.weights(L.N, L.K, "llama8b_prefill", L.name, device=dev)
        ridx = torch.as_tensor(np.sort(rng.choice(L.N, size=rows, replace=False)), device=dev)
        Wb = gen.bits(W[ridx])
        del W
        X = gen.activations(M, L.K, "llama8b_prefill", L.name, device=dev)
        midx = torch.as_tensor(np.sort(rng.choice(M, size=xrows, replace=False)), device=dev)
        Xb = gen.bits(X[midx])
        del X
        codes, scales, zeros = O.quantize_pack(Wb)
        prepared.append((L, Xb, codes, scales, zeros))
    cores = host_threads()
    flops, reps = 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        while True:
            for L, Xb, codes, scales, zeros in prepared:
                O.matmul_ref(Xb, codes, scales, zeros)
                flops += 2.0 * xrows * rows * L.K
            reps += 1
            if time.perf_counter() - t0 >= min_seconds or reps >= 5000:
                break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"{rows} output rows of each of the four layers against {xrows} of the M={M} "
                      f"activation rows, {reps} pass(es); unpack + dequantise + fp64 product "
                      f"(BLAS on {cores} threads)"}


if __name__ == "__main__":
    main()
