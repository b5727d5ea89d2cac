#!/usr/bin/env python3
"""Throughput of the W4A16 GEMM on one MI355X, on synthetic model-shaped workloads.

One step = every linear layer of one forward of the named workload (default: the
Qwen2.5-7B-shaped verify pass at M = gamma + 1 = 5: 28 layers x {qkv, o, gate_up, down} =
112 GEMMs), with all inputs resident in HBM before timing starts.  The step is captured
once into a HIP graph and replayed; W untimed replays, then K timed replays bracketed by
synchronization, timed with HIP events on the launch stream (one event between consecutive
replays, so the line carries the mean over the timed region and each replay's median and
minimum).

Printed (one JSON line): effective weight GB/s (weight bytes = 4-bit codes + fp16 scales
+ u8 zeros per 128, i.e. 0.5234375 B per weight, divided by the step time), the fraction
of the 8 TB/s HBM peak, the dominant kernel's roofline figures (its average launch duration
over the timed region, HBM traffic per launch from counters when a matching summary exists),
the oracle timed on the host cores on a bounded sample (thread count and CPU model), and the
achievable read ceilings: the library's streaming-read probe over the same byte counts, one
launch per GEMM, in a graph; the same probe as one launch over 1 GiB; and, per GEMM shape of
the step, that shape's GEMMs alone against the probe over their bytes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-ceiling]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "W4A16 verify-GEMM effective weight GB/s and % of HBM roofline at M=gamma+1"
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(ROOT, "int4_weight_only_gemm_amd", "csrc", "w4a16.hip")
KERNEL_NAME = "w4a16_kernel"           # small M: fp16 matrix cores, exact (q - z) operands
KERNEL_NAME_LARGE = "w4a16_mfma_kernel"  # M >= 64 (and large GEMMs from M = 17): bf16 matrix cores
KERNEL_NAME_NARROW = "w4a16_narrow_kernel"  # M <= 16, few tiles: one 16-column tile over all of K
# HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE passes (a text summary with
# "key: value" lines); used only while the kernel source hash and workload still match.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_w4a16_kernel_qwen2.5-7b-verify-m5.md")
CPU_SAMPLE_SECONDS = 10.0
PROBE_BLOCKS = 768  # streaming-read probe: three workgroups of 256 lanes per CU
ONE_LAUNCH_PROBE_BYTES = 1 << 30


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def graph_ms(torch, fn, stream, reps):
    """Capture fn into a HIP graph on stream and return the median replay time in ms."""
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        g.replay()
        evs[0].record(stream)
        for i in range(reps):
            g.replay()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(reps))
    del g
    return t[len(t) // 2]


def per_shape_ceilings(args, gemms, calls, stream, sink, dev):
    """For each distinct GEMM shape of the step: its GEMMs alone (every copy the step holds,
    so the weights stream from HBM as in the step) and the streaming-read probe over the same
    byte counts, one launch per GEMM, as graph replays."""
    import torch
    import int4_weight_only_gemm_amd as w4
    handle = stream.cuda_stream
    shapes = {}
    for (spec, _), call in zip(gemms, calls):
        shapes.setdefault((spec.M, spec.K, spec.N, spec.bits, spec.act4), []).append((spec, call))
    out = []
    for (M, K, N, bits, a4), items in shapes.items():
        def gemm_fn():
            for _, (fn, c) in items:
                rc = fn(*c, handle)
                if rc:
                    raise w4.W4Error(rc, fn.__name__)
        nbytes = (items[0][0].weight_bytes + 15) // 16 * 16
        region = torch.empty(nbytes * len(items) // 4, dtype=torch.int32, device=dev)
        base = region.data_ptr()

        def probe_fn():
            for i in range(len(items)):
                w4.read_probe_raw(base + i * nbytes, nbytes, sink.data_ptr(), PROBE_BLOCKS, handle)
        g_us = graph_ms(torch, gemm_fn, stream, 10) * 1e3 / len(items)
        p_us = graph_ms(torch, probe_fn, stream, 10) * 1e3 / len(items)
        del region
        wb = items[0][0].weight_bytes
        out.append({"M": M, "K": K, "N": N, "bits": bits, "a4": a4, "copies": len(items),
                    "gemm_us": round(g_us, 3), "probe_us": round(p_us, 3),
                    "gemm_gbs": round(wb / g_us / 1e3, 1), "probe_gbs": round(wb / p_us / 1e3, 1),
                    "gemm_over_probe": round(p_us / g_us, 4)})
        log(f"shape {M}x{K}x{N}: GEMM {g_us:.2f} us, probe {p_us:.2f} us per launch ({len(items)} copies)")
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(path: str = KERNEL_SOURCE) -> str:
    """Hash of the kernel source's code: comments, trailing spaces and blank lines removed,
    so that a comment-only edit keeps the counters taken on that code valid."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel, or None when no summary matches."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            m = re.match(r"^\s*-?\s*`?([a-z0-9_]+)`?\s*:\s*`?([^`\s]+)`?\s*$", line)
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256_16") != source_hash() or kv.get("workload") != workload:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen2.5-7b-verify-m5")
    ap.add_argument("--copies", type=int, default=1,
                    help="repeat the workload's GEMMs this many times with distinct weights in one step "
                         "(e.g. 512 copies of the single GEMM exceed the on-chip caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--op", choices=("gemm", "quantize"), default="gemm",
                    help="gemm: the W4A16 step (default); quantize: w4_quantize over the step's weight matrices")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--eager-steps", type=int, default=0,
                    help="only run this many eager steps (for a profiler) and print nothing else")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 5 times (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each GPU would "
              "hold a column shard of every weight matrix and compute its columns of C). "
              "Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_weight_only_gemm_amd as w4
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: 5 copies of {args.copy_probe_mib} MiB")
        return

    wl = synth.with_copies(synth.WORKLOADS[args.workload], args.copies)
    if args.op == "quantize":
        return bench_quantize(args, wl, dev)
    t0 = time.time()
    gemms = []  # (spec, device tensors, out)
    host_sample = []
    for i, spec in enumerate(wl.gemms):
        x = synth.generate(spec)
        d = {
            "A": torch.from_numpy(x.A.view(np.int16)).to(dev).view(torch.bfloat16),
            "S": torch.from_numpy(x.S.view(np.int16)).to(dev).view(torch.float16),
            "Z": torch.from_numpy(x.Z).to(dev),
        }
        if x.Wq is not None:
            d["Wq"] = torch.from_numpy(x.Wq.view(np.int32)).to(dev)
        else:
            d["Wq"] = w4.pack(torch.from_numpy(x.q).to(dev), bits=spec.bits)
        if spec.act4:  # 4-bit activations in place of the bfloat16 ones
            d["A"] = torch.from_numpy(x.Aq.view(np.int32)).to(dev)
            d["As"] = torch.from_numpy(x.As).to(dev)
        d["C"] = torch.empty((spec.M, spec.N), dtype=torch.float32, device=dev)
        gemms.append((spec, d))
        if not args.no_cpu_baseline:
            host_sample.append((spec, x))
    torch.cuda.synchronize()
    log(f"{args.workload}: {len(gemms)} GEMMs, {wl.weight_bytes / 1e9:.3f} GB of weights, "
        f"inputs ready in {time.time() - t0:.1f} s")

    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream
    lib = w4.lib()
    # each GEMM through the C-ABI entry point of its code width
    calls = [(lib.w4a4_gemm, (d["A"].data_ptr(), d["As"].data_ptr(), d["Wq"].data_ptr(), d["S"].data_ptr(),
                              d["Z"].data_ptr(), d["C"].data_ptr(), spec.M, spec.K, spec.N)) if spec.act4 else
             (lib.w8a16_gemm if spec.bits == 8 else lib.w4a16_gemm,
              (d["A"].data_ptr(), d["Wq"].data_ptr(), d["S"].data_ptr(), d["Z"].data_ptr(), d["C"].data_ptr(),
               spec.M, spec.K, spec.N)) for spec, d in gemms]

    def step():
        for fn, c in calls:
            rc = fn(*c, handle)
            if rc:
                raise w4.W4Error(rc, fn.__name__)

    # one eager step sizes the split-K workspace of this stream before capture
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()

    if args.eager_steps:
        with torch.cuda.stream(stream):
            for i in range(args.eager_steps):
                step()
                torch.cuda.synchronize()
                log(f"eager step {i + 1}/{args.eager_steps} done")
        return

    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run_step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # one HIP event between consecutive replays: the timed region is first to last event,
    # and each replay's own duration gives the median and the minimum
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(args.steps):
            run_step()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ev0, ev1 = evs[0], evs[-1]
    elapsed_ms = ev0.elapsed_time(ev1)
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    ms_min = per_step[0]
    ms_per_step = elapsed_ms / args.steps
    gbs = wl.weight_bytes / (ms_per_step * 1e-3) / 1e9
    tflops = wl.flops / (ms_per_step * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step (median {ms_median:.4f}, min {ms_min:.4f}), "
        f"{gbs:.1f} GB/s, {tflops:.2f} TFLOP/s")

    # Roofline figures of the dominant kernel.  The bound follows the step's arithmetic
    # intensity against the ridge of the two peaks (2*M flops per 0.5234375 weight bytes:
    # matrix-core-bound from M ~ 82 on); the named kernel is the one streaming most of the
    # step's weight bytes, and every GEMM kernel of the step is listed with its share of
    # those bytes.  The average launch duration is the timed region (HIP events on the launch
    # stream) divided by the GEMM launches it holds, so it covers all of the step's GEMM
    # kernels; the algorithmic bytes (or flops) per launch are the step's totals divided by
    # the same count.
    launches = args.steps * len(calls)
    avg_dur_s = elapsed_ms * 1e-3 / launches
    kinds = [w4.plan(spec.M, spec.K, spec.N, bits=spec.bits, a4=spec.act4)["kernel"] for spec, _ in gemms]
    share = {}
    for (spec, _), k in zip(gemms, kinds):
        name = KERNEL_NAME_LARGE if k == 3 else (KERNEL_NAME_NARROW if k == 8 else KERNEL_NAME)
        share[name] = share.get(name, 0) + spec.weight_bytes
    kernel = max(share, key=share.get)
    share = {name: round(b / wl.weight_bytes, 4) for name, b in share.items()}
    dtype = "bf16" if all(k == 3 for k in kinds) else ("f16" if all(k != 3 for k in kinds) else "f16+bf16")
    mfma_bound = wl.flops / wl.weight_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:  # a dense contraction, priced against the bf16 MFMA peak
        achieved = wl.flops / len(calls) / avg_dur_s / 1e12
        peak, unit, bound = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved = wl.weight_bytes / len(calls) / avg_dur_s / 1e9
        peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
    log(f"dominant kernel: {launches} launches, avg {avg_dur_s * 1e6:.2f} us, {achieved:.1f} {unit}")

    traffic = read_traffic(args.workload)

    ceiling = None
    if not args.no_ceiling:
        # Achievable HBM read rate for this step's byte counts: the streaming-read probe reads
        # one buffer per GEMM holding exactly that GEMM's weight bytes (codes, scales, zeros),
        # one launch per GEMM, captured and replayed like the step.
        sizes = [(spec.weight_bytes + 15) // 16 * 16 for spec, _ in gemms]
        region = torch.empty(sum(sizes) // 4, dtype=torch.int32, device=dev)
        sink = torch.empty((PROBE_BLOCKS, 4), dtype=torch.int32, device=dev)
        base, offs = region.data_ptr(), []
        for n in sizes:
            offs.append(base)
            base += n

        def probe_step():
            for ptr, n in zip(offs, sizes):
                w4.read_probe_raw(ptr, n, sink.data_ptr(), PROBE_BLOCKS, handle)

        with torch.cuda.stream(stream):
            probe_step()
        torch.cuda.synchronize()
        pgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph, stream=stream):
            probe_step()
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                pgraph.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for _ in range(args.steps):
                pgraph.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        probe_ms = ev0.elapsed_time(ev1) / args.steps
        cgbs = sum(sizes) / (probe_ms * 1e-3) / 1e9
        ceiling = {"kind": "streaming-read probe", "value": round(cgbs, 2), "unit": "GB/s",
                   "frac_of_peak": round(cgbs / HBM_PEAK_GBS, 4),
                   "gemm_over_ceiling": round(gbs / cgbs, 4),
                   "ms_per_step": round(probe_ms, 5), "launches_per_step": len(sizes), "blocks": PROBE_BLOCKS}
        log(f"streaming-read ceiling: {cgbs:.1f} GB/s ({probe_ms:.4f} ms per step); GEMM step at "
            f"{100 * gbs / cgbs:.1f}% of it")
        del pgraph, region
        # The same probe as one launch over 1 GiB: the streaming rate without per-launch costs.
        big = ONE_LAUNCH_PROBE_BYTES
        bufb = torch.empty(big // 4, dtype=torch.int32, device=dev)
        with torch.cuda.stream(stream):
            for _ in range(2):
                w4.read_probe_raw(bufb.data_ptr(), big, sink.data_ptr(), PROBE_BLOCKS, handle)
            ev0.record(stream)
            for _ in range(5):
                w4.read_probe_raw(bufb.data_ptr(), big, sink.data_ptr(), PROBE_BLOCKS, handle)
            ev1.record(stream)
        torch.cuda.synchronize()
        one_ms = ev0.elapsed_time(ev1) / 5
        ceiling["one_launch"] = {"bytes": big, "value": round(big / (one_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                                 "ms": round(one_ms, 4), "blocks": PROBE_BLOCKS}
        ceiling["one_launch"]["frac_of_peak"] = round(ceiling["one_launch"]["value"] / HBM_PEAK_GBS, 4)
        log(f"one-launch probe over {big / 2**30:.0f} GiB: {ceiling['one_launch']['value']} GB/s")
        del bufb
        # Per GEMM shape of the step: the GEMMs of that shape alone, and the probe over their
        # byte counts, each captured and replayed like the step (one launch per GEMM).
        ceiling["per_shape"] = per_shape_ceilings(args, gemms, calls, stream, sink, dev)

    cpu = None
    if not args.no_cpu_baseline:
        # The oracle as it stands, on the host cores, over whole GEMMs of this workload taken
        # in step order (wrapping round) until CPU_SAMPLE_SECONDS have passed.
        import oracle
        orc = oracle.get()
        threads = len(os.sched_getaffinity(0))
        t1 = time.perf_counter()
        nbytes, done = 0, 0
        while time.perf_counter() - t1 < CPU_SAMPLE_SECONDS:
            spec, x = host_sample[done % len(host_sample)]
            Wq = x.Wq if x.Wq is not None else (orc.pack8(x.q) if spec.bits == 8 else orc.pack(x.q))
            if spec.act4:
                orc.gemm_a4(x.Aq, x.As, Wq, x.S, x.Z, threads=threads)
            else:
                orc.gemm(x.A, Wq, x.S, x.Z, threads=threads, bits=spec.bits)
            nbytes += spec.weight_bytes
            done += 1
        dt = time.perf_counter() - t1
        cpu = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"{done} GEMMs of {args.workload} in step order, wrapping round the step "
                         f"({done / len(host_sample):.2f} steps of {len(host_sample)} GEMMs; every output element), "
                         f"{nbytes / 1e6:.1f} MB of weights in {dt:.2f} s"}
        log(f"cpu oracle: {cpu['value']} GB/s on {threads} threads ({dt:.2f} s)")

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "ms_per_step_min": round(ms_min, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tflops": round(tflops, 3),
        "config": {
            "workload": args.workload,
            "variant": "+".join(sorted({"w4a4" if s.act4 else f"w{s.bits}a16" for s, _ in gemms})),
            "gemms_per_step": len(gemms),
            "copies": args.copies,
            "M": sorted({s.M for s, _ in gemms}),
            "weight_bytes_per_step": wl.weight_bytes,
            "hip_graph": graph is not None,
        },
        "roofline": {
            "bound": bound,
            "kernel": kernel,
            "weight_byte_share": share,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_dur_s * 1e6, 3),
            "launches_timed": launches,
        },
        "cpu_baseline": cpu,
        "ceiling": ceiling,
    }
    print(json.dumps(out), flush=True)


def bench_quantize(args, wl, dev):
    """w4_quantize over every weight matrix of the workload (binary16 weights drawn on the
    device, N(0, 0.02^2) with a per-matrix seed), captured in a HIP graph like the GEMM step.
    Bytes moved per weight: 2 (binary16 read) + 0.5234375 (storage format written)."""
    import torch
    import int4_weight_only_gemm_amd as w4

    t0 = time.time()
    mats = []
    for spec in wl.gemms:
        gen = torch.Generator(device=dev)
        gen.manual_seed(int(np.random.SeedSequence(list(spec.seed) + [2]).generate_state(1)[0]))
        W = torch.randn((spec.K, spec.N), dtype=torch.float16, device=dev, generator=gen) * 0.02
        outs = (torch.empty((spec.K // 8, spec.N), dtype=torch.int32, device=dev),
                torch.empty((spec.K // 128, spec.N), dtype=torch.float16, device=dev),
                torch.empty((spec.K // 128, spec.N), dtype=torch.uint8, device=dev))
        mats.append((spec, W, outs))
    torch.cuda.synchronize()
    nbytes = sum(spec.K * spec.N * 2 + spec.weight_bytes for spec, _, _ in mats)
    log(f"{args.workload}: {len(mats)} weight matrices, {nbytes / 1e9:.3f} GB moved per step, "
        f"inputs ready in {time.time() - t0:.1f} s")
    stream = torch.cuda.Stream(device=dev)
    handle = stream.cuda_stream

    def step():
        for spec, W, (Wq, S, Z) in mats:
            w4.quantize_raw(W.data_ptr(), Wq.data_ptr(), S.data_ptr(), Z.data_ptr(), spec.K, spec.N, handle)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    launches = args.steps * len(mats)
    avg_us = ev0.elapsed_time(ev1) * 1e3 / launches
    log(f"timed {args.steps} steps: {ms:.4f} ms/step, {gbs:.1f} GB/s, avg launch {avg_us:.2f} us")

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's quantizer on the host, over the step's matrices in order (wrapping
        # round), on host copies of the same weights, until CPU_SAMPLE_SECONDS have passed
        import oracle
        orc = oracle.get()
        sample = mats[:min(len(mats), 8)]  # the first layers' matrices, copied before timing
        host = [(spec, W.cpu().numpy().view(np.uint16)) for spec, W, _ in sample]
        t1 = time.perf_counter()
        done, moved = 0, 0
        while time.perf_counter() - t1 < CPU_SAMPLE_SECONDS:
            spec, Wh = host[done % len(host)]
            orc.quantize(Wh)
            moved += spec.K * spec.N * 2 + spec.weight_bytes
            done += 1
        dt = time.perf_counter() - t1
        cpu = {"value": round(moved / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} quantizations of the first {len(host)} weight matrices of {args.workload}, "
                         f"wrapping round (single-threaded oracle quantizer), {moved / 1e6:.1f} MB moved in {dt:.2f} s"}
        log(f"cpu oracle quantizer: {cpu['value']} GB/s")

    out = {
        "metric": "w4_quantize GB/s (binary16 weights read + storage format written)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "op": "quantize", "matrices_per_step": len(mats),
                   "bytes_per_step": nbytes, "hip_graph": True},
        "roofline": {"bound": "hbm", "kernel": "w4_quantize_kernel", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(avg_us, 3), "launches_timed": launches},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
