#!/usr/bin/env python3
"""Benchmark of one absorbed-MLA decode step on one MI355X.

A step is one call of the whole hot path (query absorption, split-context
attention over the latent + RoPE cache, log-sum-exp combine, W_UV
up-projection) on one batch of synthetic DeepSeek-V2-shaped inputs that are
already resident in HBM.  To keep the 256 MB Infinity Cache from serving the
cache and weights, steps rotate over enough distinct device copies
("layers") of the cache and weights to exceed 1 GiB.

Prints ONE JSON line on stdout (progress goes to stderr).  `value` is the
algorithmic attention TFLOP/s of the whole step (FLOPs counted as 4 h d_c +
2 h d_r + h per visible (query, cached token) pair plus 2 h d_h d_c per query
row for each of the two projections, softmax excluded); `cache_gbps` is the
latent + RoPE cache bytes per step over the step time.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode attention TFLOP/s + latent-cache GB/s (h=128,d_c=512) @ T=4K..128K"
HBM_GBPS = 8000.0          # MI355X HBM3E peak
MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
MFMA_F32_TFLOPS = 157.3
MIN_ROTATION_BYTES = 1 << 30


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def chunk_count(wl, splits, chunk, num_cus):
    """Chunks of the step: batch * splits for a fixed chunking; for one
    planned on the device ((0, 0) from mla_decode_split_plan) the same choice
    the kernels make from the context lengths, redone here for the byte
    counts."""
    if splits > 0:
        return wl.batch * splits
    lens = [min(max(int(L), 0), int(wl.max_len)) for L in wl.lens]
    total = sum(lens)
    target = max(1, num_cus // (wl.n_q * (wl.h // 64)))

    def length(parts):
        c = -(-(-(-total // max(parts, 1))) // 32) * 32
        return min(max(c, 128), 1024 * 32)

    def count(c):
        return sum(-(-L // c) for L in lens)
    parts = target
    for _ in range(3):
        c = length(parts)
        n = count(c)
        if n <= target or c == 1024 * 32:
            return n
        parts -= n - target
        if parts < 1:
            break
    return count(length(target - wl.batch))


def counts(wl, chunks):
    """Algorithmic bytes and FLOPs of one step, per kernel (`chunks`: chunk
    results of one query token, over all sequences)."""
    el = 2 if wl.dtype == "bf16" else 4
    R = wl.rows
    pairs = wl.visible_pairs()
    per_pair = 4 * wl.h * wl.d_c + 2 * wl.h * wl.d_r + wl.h
    proj_flops = 2 * R * wl.h * wl.d_h * wl.d_c
    w_bytes = wl.h * wl.d_h * wl.d_c * el
    cache_bytes = wl.cache_tokens() * (wl.d_c + wl.d_r) * el
    # chunk partials: bf16 latent + fp32 lse on the bf16 fast path, fp32 otherwise
    part_bytes = chunks * wl.n_q * wl.h * (wl.d_c * el + 4)
    absorb_bytes = w_bytes + R * wl.h * (wl.d_h * el + wl.d_c * 2)
    return {
        "q_absorb": dict(bytes=absorb_bytes, flops=proj_flops),
        "split_attn": dict(bytes=cache_bytes, flops=pairs * per_pair, partial_bytes=part_bytes),
        "combine": dict(bytes=part_bytes + R * wl.h * wl.d_c * 2, flops=0),
        "up_project": dict(bytes=w_bytes + R * wl.h * (wl.d_c * 2 + wl.d_h * el), flops=proj_flops),
        # chunk merge fused with the up-projection (bf16 fast path)
        "finish": dict(bytes=part_bytes + w_bytes + R * wl.h * wl.d_h * el, flops=proj_flops),
        "step": dict(bytes=cache_bytes + 2 * w_bytes, flops=pairs * per_pair + 2 * proj_flops,
                     cache_bytes=cache_bytes),
    }


def kernel_roofline(name, c, avg_s, dtype):
    """Bound, achieved and peak for one kernel from its algorithmic counts."""
    peak_flops = MFMA_BF16_TFLOPS if dtype == "bf16" else MFMA_F32_TFLOPS
    ridge = peak_flops * 1e12 / (HBM_GBPS * 1e9)
    ai = c["flops"] / c["bytes"] if c["bytes"] else float("inf")
    if c["flops"] and ai > ridge:
        achieved = c["flops"] / avg_s / 1e12
        return dict(bound="mfma", achieved=achieved, peak=peak_flops, unit="TFLOP/s",
                    frac=achieved / peak_flops)
    achieved = c["bytes"] / avg_s / 1e9
    return dict(bound="hbm", achieved=achieved, peak=HBM_GBPS, unit="GB/s", frac=achieved / HBM_GBPS)


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    from mla_latent_cache_absorbed_amd.profiling import TRAFFIC_FILE, source_digest
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        e = t[kernel][workload]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("source_digest") != source_digest(kernel):
        return None
    return e.get("bytes_per_launch")


class Layers:
    """Distinct device copies of the cache, queries and weights of a workload."""

    def __init__(self, dw, n):
        import torch
        keys = ("q", "q_r", "latent_pool", "rope_pool", "w_uk", "w_uv")
        self.sets = [dict(dw.t)]
        for _ in range(n - 1):
            d = dict(dw.t)
            for k in keys:
                d[k] = dw.t[k].clone()
            self.sets.append(d)
        torch.cuda.synchronize()

    def __len__(self):
        return len(self.sets)


def layer_bytes(wl):
    el = 2 if wl.dtype == "bf16" else 4
    return el * (wl.num_pages * wl.page_size * (wl.d_c + wl.d_r) + 2 * wl.h * wl.d_h * wl.d_c)


def prepared_calls(dw, layers):
    """The C entry point and one argument tuple per layer set, marshalled
    once: every set goes through the checked binding first (shapes, dtypes,
    device, contiguity), and the timed loop then calls mla_decode_run with
    the same pointers directly.  The per-call checks in Python take about as
    long as a whole T=4K step on the GPU, so in the loop they would set the
    launch rate instead of the kernels."""
    import torch
    from mla_latent_cache_absorbed_amd import binding
    stream = torch.cuda.current_stream().cuda_stream
    wl = dw.wl
    calls = []
    for t in layers.sets:
        dw.run(**t)
        calls.append((dw.dec.plan, wl.batch, wl.n_q, dw.max_len, int(t["latent_pool"].shape[0]),
                      t["q"].data_ptr(), t["q_r"].data_ptr(), t["latent_pool"].data_ptr(),
                      t["rope_pool"].data_ptr(), t["page_table"].data_ptr(), t["context_lens"].data_ptr(),
                      t["w_uk"].data_ptr(), t["w_uv"].data_ptr(), dw.out.data_ptr(), dw.ws.data_ptr(),
                      dw.ws.numel() * dw.ws.element_size(), stream))
    torch.cuda.synchronize()
    return binding.lib().mla_decode_run, calls


def time_steps(dw, layers, steps, warmup, per_kernel):
    """Average step time (s); with per_kernel, also per-kernel averages (s)."""
    import torch
    from mla_latent_cache_absorbed_amd import binding
    n = len(layers)
    run, calls = prepared_calls(dw, layers)
    for i in range(warmup):
        binding.raise_for_status(run(*calls[i % n]))
    torch.cuda.synchronize()
    if per_kernel:
        binding.mla_decode_enable_timing(dw.dec.plan, steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    status = 0
    for i in range(steps):
        status = min(status, run(*calls[(warmup + i) % n]))  # failures are negative
    end.record()
    binding.raise_for_status(status)
    torch.cuda.synchronize()
    step_s = start.elapsed_time(end) / 1e3 / steps
    kernels = None
    if per_kernel:
        ms, runs = binding.mla_decode_read_timing(dw.dec.plan)
        binding.mla_decode_enable_timing(dw.dec.plan, 0)
        kernels = {k: v / 1e3 / runs for k, v in ms.items()}
        if kernels.get("up_project") == 0:  # merge and up-projection ran as one kernel
            kernels = {"q_absorb": kernels["q_absorb"], "split_attn": kernels["split_attn"],
                       "finish": kernels["combine"]}
    return step_s, kernels


def achievable_peaks():
    """What plain library work reaches on this GPU, for context beside the
    vendor peaks: a 1 GiB device-to-device copy (read + write bytes) and a
    bf16 8192^3 GEMM (hipBLASLt through torch), each timed with events."""
    import torch
    res = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    res["copy_gbps"] = 2 * n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    res["gemm_bf16_tflops"] = 2 * m ** 3 * reps / (e0.elapsed_time(e1) / 1e3) / 1e12
    res["what"] = ("1 GiB device-to-device copy (torch copy_, read + write bytes) and a bf16 "
                   "8192x8192x8192 torch.mm, 10 timed repetitions each")
    return res


def time_graph(dw, layers, steps, warmup):
    """Average step time (s) of the same steps replayed from one HIP graph
    that holds one step per layer set (the launches of mla_decode_run are
    captured from torch's current stream)."""
    import torch
    n = len(layers)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            dw.run(**layers.sets[i])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            dw.run(**layers.sets[i])
    for _ in range(max(1, warmup // n)):
        graph.replay()
    reps = max(1, math.ceil(steps / n))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / 1e3 / (reps * n)


def cpu_baseline(wl, target_s=15.0):
    """Time the fp64 oracle (explicit K/V form, as it stands) on a bounded
    sample of the workload: whole decode of a subset of (sequence, head)
    pairs, sized for about target_s seconds of CPU work."""
    import numpy as np
    import oracle
    from mla_latent_cache_absorbed_amd import inputs
    prob = oracle.Problem(**inputs.oracle_problem_kwargs(wl))
    threads = oracle.num_threads()
    all_pairs = [(b, i) for b in range(wl.batch) for i in range(wl.h)]

    def run(n):
        pairs = all_pairs[:n]
        t = time.perf_counter()
        oracle.decode_explicit(prob, pairs)
        return time.perf_counter() - t, pairs

    n = min(len(all_pairs), max(1, threads))
    dt, pairs = run(n)
    if dt < target_s / 3:
        n = int(min(len(all_pairs), max(n, round(n * target_s / max(dt, 1e-3)))))
        dt, pairs = run(n)
    reps = 1
    if dt < target_s / 3:  # the whole workload is short: repeat it for a steadier figure
        reps = max(1, int(round(target_s / max(dt, 1e-3))))
        t = time.perf_counter()
        for _ in range(reps):
            run(n)
        dt = (time.perf_counter() - t) / reps
    per_pair = 4 * wl.d_c + 2 * wl.d_r + 1
    flops = 0
    for b, _ in pairs:
        L = int(wl.lens[b])
        flops += sum(L - wl.n_q + m + 1 for m in range(wl.n_q)) * per_pair
        flops += wl.n_q * 2 * 2 * wl.d_h * wl.d_c
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=min(threads, len(pairs)),
                kind="oracle",
                sample="explicit fp64 oracle (per-head K/V rebuilt, textbook softmax) on %d of "
                       "%d (sequence, head) pairs of %s, %.2f s wall per pass, mean of %d pass(es)"
                       % (len(pairs), len(all_pairs), wl.name, dt, reps),
                seconds=dt)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ds2_t4k")
    ap.add_argument("--extra", default="ds2_t32k,ds2_t128k,ds2_paged_b32,ds2_mtp_b16",
                    help="comma-separated further workloads whose steps and split kernel are "
                         "also measured ('' = none)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the copy and GEMM measurements of achievable peaks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="0 = enough for 1 GiB")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run plain device-to-device copies of MB MiB (the reference kernel "
                         "for scaling HBM byte counters) and print their size")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_latent_cache_absorbed_amd import inputs
    from mla_latent_cache_absorbed_amd.runner import DeviceWorkload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": args.steps}))
        return

    def measure(name, steps, warmup):
        wl = inputs.make(name)
        dw = DeviceWorkload(wl)
        n_layers = args.layers or max(2, min(60, math.ceil(MIN_ROTATION_BYTES / layer_bytes(wl))))
        layers = Layers(dw, n_layers)
        splits, chunk = dw.split_plan()
        log("%s: %d layers rotated (%.0f MB each), %d chunks of %d tokens" %
            (name, n_layers, layer_bytes(wl) / 1e6, splits, chunk))
        step_s, _ = time_steps(dw, layers, steps, warmup, per_kernel=False)
        graph_s = time_graph(dw, layers, steps, warmup)
        log("%s: step %.2f us eager, %.2f us replayed from a HIP graph" % (name, step_s * 1e6, graph_s * 1e6))
        _, kern = time_steps(dw, layers, steps, 2, per_kernel=True)
        c = counts(wl, chunk_count(wl, splits, chunk, torch.cuda.get_device_properties(0).multi_processor_count))
        del layers
        return wl, dw, c, step_s, graph_s, kern, splits, chunk, n_layers

    wl, dw, c, step_s, graph_s, kern, splits, chunk, n_layers = measure(args.workload, args.steps,
                                                                       args.warmup)
    log("step %.2f us; kernels (us): %s" % (step_s * 1e6, {k: round(v * 1e6, 2) for k, v in kern.items()}))

    rooflines = {k: kernel_roofline(k, c[k], kern[k], wl.dtype) for k in kern}
    dominant = max(kern, key=lambda k: kern[k])
    roof = dict(rooflines[dominant])
    roof["kernel"] = dominant
    roof["avg_us"] = kern[dominant] * 1e6
    traffic = measured_traffic(dominant, wl.name)
    roof["traffic"] = traffic
    roof = {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel", "avg_us")}

    out = {
        "metric": METRIC,
        "value": c["step"]["flops"] / step_s / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "graph_ms_per_step": graph_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q": wl.n_q,
                   "context": int(wl.max_len), "h": wl.h, "d_c": wl.d_c, "d_r": wl.d_r,
                   "d_h": wl.d_h, "page_size": wl.page_size, "splits": splits,
                   "chunk_len": chunk, "layers_rotated": n_layers},
        "cache_gbps": c["step"]["cache_bytes"] / step_s / 1e9,
        "roofline": roof,
        # the whole step against the same HBM peak: the bytes the method must
        # move per step (cache read once, W_UK and W_UV once) over its wall time
        "step_hbm": dict(algorithmic_bytes=c["step"]["bytes"], achieved=c["step"]["bytes"] / step_s / 1e9,
                         peak=HBM_GBPS, unit="GB/s", frac=c["step"]["bytes"] / step_s / 1e9 / HBM_GBPS),
        "kernels": {k: dict(avg_us=kern[k] * 1e6, **rooflines[k]) for k in kern},
    }

    def split_entry(wl2, c2, kern2, s2, ch2, nl2, step2=None, graph2=None):
        k = "split_attn"
        t_split = kern2[k]
        e = dict(split_us=t_split * 1e6, splits=s2, chunk_len=ch2, layers_rotated=nl2,
                 cache_gbps=c2["split_attn"]["bytes"] / t_split / 1e9,
                 cache_plus_partials_gbps=(c2["split_attn"]["bytes"] + c2["split_attn"]["partial_bytes"])
                 / t_split / 1e9,
                 tflops=c2["split_attn"]["flops"] / t_split / 1e12,
                 kernels_us={kk: v * 1e6 for kk, v in kern2.items()},
                 roofline=dict(kernel_roofline(k, c2[k], t_split, wl2.dtype),
                               traffic=measured_traffic(k, wl2.name)))
        if step2 is not None:
            e.update(step_us=step2 * 1e6, step_tflops=c2["step"]["flops"] / step2 / 1e12,
                     step_hbm_gbps=c2["step"]["bytes"] / step2 / 1e9, graph_step_us=graph2 * 1e6)
        return e

    sweep = {}
    for name in [n for n in args.extra.split(",") if n]:
        wl2, dw2, c2, step2, graph2, kern2, s2, ch2, nl2 = measure(name, max(10, args.steps // 2), 5)
        sweep[wl2.name] = split_entry(wl2, c2, kern2, s2, ch2, nl2, step2, graph2)
        log("%s: step %.2f us; kernels (us): %s" % (name, step2 * 1e6,
                                                   {k: round(v * 1e6, 2) for k, v in kern2.items()}))
        del dw2
    if sweep:
        out["sweep"] = sweep
        if "ds2_t32k" in sweep:  # the point the split kernel's roofline bar is set at
            out["split_kernel_ds2_t32k"] = dict(sweep["ds2_t32k"])

    if not args.no_achievable:
        out["achievable"] = achievable_peaks()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
