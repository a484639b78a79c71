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

The headline workload is B=1, T=32K (the split kernel's roofline bar point);
the other DeepSeek-V2-shaped configurations are measured in `sweep`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

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


def stats(values):
    """mean, median, p10, p90 (nearest-rank) and count of a list of numbers."""
    v = sorted(values)
    n = len(v)

    def rank(q):
        return v[min(n - 1, max(0, int(math.ceil(q * n)) - 1))]
    return dict(mean=sum(v) / n, median=rank(0.5), p10=rank(0.1), p90=rank(0.9), n=n)


def step_distribution(dw, layers, n):
    """n more steps, each between two events recorded on torch's current
    stream (the stream the library launches on): per-step seconds."""
    import torch
    from mla_latent_cache_absorbed_amd import binding
    run, calls = prepared_calls(dw, layers)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    status = 0
    ev[0].record()
    for i in range(n):
        status = min(status, run(*calls[i % len(calls)]))
        ev[i + 1].record()
    binding.raise_for_status(status)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(n)]


def kernel_distribution(dw, layers, n):
    """n more steps with every kernel's own start and stop recorded by its
    dispatch (events on the kernel's stream): per-run seconds of each kernel."""
    import torch
    from mla_latent_cache_absorbed_amd import binding
    run, calls = prepared_calls(dw, layers)
    binding.mla_decode_enable_timing(dw.dec.plan, n)
    torch.cuda.synchronize()
    status = 0
    for i in range(n):
        status = min(status, run(*calls[i % len(calls)]))
    binding.raise_for_status(status)
    per_run = binding.mla_decode_read_timing_runs(dw.dec.plan, n)
    binding.mla_decode_enable_timing(dw.dec.plan, 0)
    out = {}
    for r in per_run:
        if r.get("up_project", 0) == 0:  # merge and up-projection ran as one kernel
            r = {"q_absorb": r["q_absorb"], "split_attn": r["split_attn"], "finish": r["combine"]}
        for k, v in r.items():
            out.setdefault(k, []).append(v / 1e3)
    return out


def launch_floor(dw, layers, n):
    """Per-kernel times of the same plan and grids with every context length
    set to 1: all split work-groups but one find no visible token and leave
    at once, so the split kernel's time is its launch-and-drain floor at this
    grid (the absorb and finish kernels do their usual work)."""
    import copy
    import torch
    floor = copy.copy(layers)
    floor.sets = []
    for s in layers.sets:
        d = dict(s)
        d["context_lens"] = torch.ones_like(s["context_lens"])
        floor.sets.append(d)
    return kernel_distribution(dw, floor, n)


def measure_oproj(rows, runs, warmup):
    """The output projection u = [o_1; ...; o_h] W^O at DeepSeek-V2 width
    (k = 16384, d = 5120) for `rows` query rows: per-call events on the
    launch stream over `runs` calls, rotating over enough device copies of
    W^O (168 MB each) to exceed 1 GiB, so that the weight comes from HBM."""
    import torch
    from mla_latent_cache_absorbed_amd import binding, inputs
    case = inputs.make_oproj(rows, seed=320 + rows)
    k, d = case["k"], case["d"]
    o = torch.from_numpy(case["o"].reshape(rows, k).view(np.int16)).view(torch.bfloat16).cuda()
    w0 = torch.from_numpy(np.ascontiguousarray(case["w_o"].T).view(np.int16)).view(torch.bfloat16).cuda()
    n = max(2, math.ceil(MIN_ROTATION_BYTES / (w0.numel() * 2)))
    ws = [w0] + [w0.clone() for _ in range(n - 1)]
    u = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    need = binding.mla_oproj_workspace_size(rows, k, d)
    part = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    L = binding.lib()
    # argument tuples marshalled once (the checked wrapper's Python work per
    # call would be comparable to the call itself)
    binding.mla_oproj_run(rows, k, d, o, ws[0], u, part, need, stream=stream)
    calls = [(rows, k, d, binding.MLA_DTYPE_BF16, binding.MLA_DTYPE_BF16, o.data_ptr(), w.data_ptr(),
              u.data_ptr(), part.data_ptr(), need, stream) for w in ws]
    for i in range(warmup):
        binding.raise_for_status(L.mla_oproj_run(*calls[i % n]))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * runs)]
    torch.cuda.synchronize()
    status = 0
    for i in range(runs):
        ev[2 * i].record()
        status = min(status, L.mla_oproj_run(*calls[i % n]))
        ev[2 * i + 1].record()
    binding.raise_for_status(status)
    torch.cuda.synchronize()
    t = stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) / 1e3 for i in range(runs)])
    algo_bytes = 2 * (k * d + rows * k + rows * d)
    flops = 2 * rows * k * d
    del ws, w0
    return dict(rows=rows, k=k, d_model=d, slices=max(1, need // (rows * d * 4)), layers_rotated=n,
                us={kk: t[kk] * 1e6 for kk in ("mean", "median", "p10", "p90")}, runs=t["n"],
                algorithmic_bytes=algo_bytes, tflops=flops / t["median"] / 1e12,
                roofline=dict(bound="hbm", achieved=algo_bytes / t["median"] / 1e9, peak=HBM_GBPS, unit="GB/s",
                              frac=algo_bytes / t["median"] / 1e9 / HBM_GBPS,
                              traffic=measured_traffic("oproj", "oproj_r%d" % rows),
                              what="median over the runs of one call (partial kernel + slice sum)"))


def measure_projections(rows, runs, warmup):
    """The current token's projections at DeepSeek-V2 widths (d_model 5120,
    d_c 512, d_r 64, d_qc 1536, 128 heads of 128) for `rows` new tokens: the
    cache append (into a 512-page pool), the query side, and both in one
    call (mla_token_project_run), each timed per call with events on the
    launch stream over `runs` calls, rotating over enough device copies of
    its weights to exceed 1 GiB."""
    import torch
    from mla_latent_cache_absorbed_amd import binding, inputs
    case = inputs.make_projections(rows, seed=480 + rows)
    d_model, d_c, d_r, d_qc, h, d_h = (case[k] for k in ("d_model", "d_c", "d_r", "d_qc", "h", "d_h"))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    x = dev(case["x"])
    stream = torch.cuda.current_stream().cuda_stream
    L = binding.lib()

    def timed(calls, fn):
        for i in range(warmup):
            binding.raise_for_status(fn(*calls[i % len(calls)]))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * runs)]
        torch.cuda.synchronize()
        status = 0
        for i in range(runs):
            ev[2 * i].record()
            status = min(status, fn(*calls[i % len(calls)]))
            ev[2 * i + 1].record()
        binding.raise_for_status(status)
        torch.cuda.synchronize()
        return stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) / 1e3 for i in range(runs)])

    def record(t, algo_bytes, flops, n):
        return dict(rows=rows, us={kk: t[kk] * 1e6 for kk in ("mean", "median", "p10", "p90")}, runs=t["n"],
                    weight_copies=n, algorithmic_bytes=algo_bytes, tflops=flops / t["median"] / 1e12,
                    roofline=dict(bound="hbm", achieved=algo_bytes / t["median"] / 1e9, peak=HBM_GBPS, unit="GB/s",
                                  frac=algo_bytes / t["median"] / 1e9 / HBM_GBPS,
                                  what="median over the runs of one call"))

    out = {}
    # cache append: one token per row at distinct positions of one sequence
    page_size, pages = 64, 512
    table = torch.arange(pages, dtype=torch.int32, device="cuda").reshape(1, pages)
    seq = torch.zeros(rows, dtype=torch.int32, device="cuda")
    pos = torch.from_numpy(np.random.default_rng(481).choice(pages * page_size, rows, replace=False)
                           .astype(np.int32)).cuda()
    lat = torch.zeros((pages, page_size, d_c), dtype=torch.bfloat16, device="cuda")
    rp = torch.zeros((pages, page_size, d_r), dtype=torch.bfloat16, device="cuda")
    w_bytes = (d_c + d_r) * d_model * 2
    n = max(2, math.ceil(MIN_ROTATION_BYTES / w_bytes))
    w0 = (dev(case["w_dkv"]), dev(case["w_kr"]))
    ws = [w0] + [(w0[0].clone(), w0[1].clone()) for _ in range(n - 1)]
    need = binding.mla_cache_append_workspace_size(rows, d_model, d_c, d_r)
    work = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    calls = [(rows, d_model, d_c, d_r, binding.MLA_DTYPE_BF16, x.data_ptr(), a.data_ptr(), b.data_ptr(),
              seq.data_ptr(), pos.data_ptr(), table.data_ptr(), pages, page_size, pages, lat.data_ptr(),
              rp.data_ptr(), None, 10000.0, work.data_ptr(), need, stream) for a, b in ws]
    t = timed(calls, L.mla_cache_append_run)
    out["cache_append"] = record(t, w_bytes + rows * d_model * 2 + rows * (d_c + d_r) * 2,
                                 2 * rows * d_model * (d_c + d_r), n)
    del ws, lat, rp
    # query side
    q = torch.empty((rows, h, d_h), dtype=torch.bfloat16, device="cuda")
    q_r = torch.empty((rows, h, d_r), dtype=torch.bfloat16, device="cuda")
    qpos = torch.from_numpy(np.random.default_rng(482).integers(0, 131072, rows).astype(np.int32)).cuda()
    w_bytes = (d_qc * d_model + h * (d_h + d_r) * d_qc) * 2
    n = max(2, math.ceil(MIN_ROTATION_BYTES / w_bytes))
    w0 = (dev(case["w_dq"]), dev(case["w_uq"]), dev(case["w_qr"]))
    ws = [w0] + [tuple(w.clone() for w in w0) for _ in range(n - 1)]
    need = binding.mla_query_project_workspace_size(rows, d_model, d_qc, h, d_h, d_r)
    work = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    calls = [(rows, d_model, d_qc, h, d_h, d_r, binding.MLA_DTYPE_BF16, x.data_ptr(), a.data_ptr(), b.data_ptr(),
              c.data_ptr(), qpos.data_ptr(), q.data_ptr(), q_r.data_ptr(), None, 10000.0, work.data_ptr(), need,
              stream) for a, b, c in ws]
    t = timed(calls, L.mla_query_project_run)
    out["query_project"] = record(t, w_bytes + rows * d_model * 2 + rows * h * (d_h + d_r) * 2,
                                  2 * rows * (d_qc * d_model + h * (d_h + d_r) * d_qc), n)
    del ws
    # both in one call (mla_token_project_run): the same rows, positions and
    # pools as the cache append above
    lat = torch.zeros((pages, page_size, d_c), dtype=torch.bfloat16, device="cuda")
    rp = torch.zeros((pages, page_size, d_r), dtype=torch.bfloat16, device="cuda")
    w_bytes = ((d_c + d_r + d_qc) * d_model + h * (d_h + d_r) * d_qc) * 2
    n = max(2, math.ceil(MIN_ROTATION_BYTES / w_bytes))
    w0 = tuple(dev(case[k]) for k in ("w_dkv", "w_kr", "w_dq", "w_uq", "w_qr"))
    ws = [w0] + [tuple(w.clone() for w in w0) for _ in range(n - 1)]
    need = binding.mla_token_project_workspace_size(rows, d_model, d_c, d_r, d_qc, h, d_h)
    work = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    calls = [(rows, d_model, d_c, d_r, d_qc, h, d_h, binding.MLA_DTYPE_BF16, x.data_ptr()) +
             tuple(w.data_ptr() for w in ww) +
             (seq.data_ptr(), pos.data_ptr(), table.data_ptr(), pages, page_size, pages, lat.data_ptr(),
              rp.data_ptr(), q.data_ptr(), q_r.data_ptr(), None, 10000.0, work.data_ptr(), need, stream)
             for ww in ws]
    t = timed(calls, L.mla_token_project_run)
    out["token_project"] = record(t, w_bytes + rows * d_model * 2 + rows * (d_c + d_r + h * (d_h + d_r)) * 2,
                                  2 * rows * ((d_c + d_r + d_qc) * d_model + h * (d_h + d_r) * d_qc), n)
    del ws, lat, rp
    return out


def measure_prefill(T, runs, warmup, h=128):
    """Prefill (keys and values rebuilt, causal attention) of a T-token
    prompt at DeepSeek-V2 head shapes: per-call events on the launch stream
    over `runs` calls."""
    import torch
    from mla_latent_cache_absorbed_amd import binding, inputs
    case = inputs.make_prefill(T, h=h, seed=560)
    d_c, d_r, d_h = case["d_c"], case["d_r"], case["d_h"]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    t = {k: dev(case[k]) for k in ("latent", "rope", "q", "q_r", "w_uk", "w_uv")}
    out = torch.empty((T, h, d_h), dtype=torch.bfloat16, device="cuda")
    need = binding.mla_prefill_workspace_size(T, h, d_h)
    work = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    L = binding.lib()
    args = (T, h, d_c, d_r, d_h, binding.MLA_DTYPE_BF16, binding.MLA_DTYPE_BF16, 0.0, t["latent"].data_ptr(),
            t["rope"].data_ptr(), t["q"].data_ptr(), t["q_r"].data_ptr(), t["w_uk"].data_ptr(), t["w_uv"].data_ptr(),
            out.data_ptr(), work.data_ptr(), need, stream)
    for _ in range(warmup):
        binding.raise_for_status(L.mla_prefill_run(*args))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * runs)]
    torch.cuda.synchronize()
    status = 0
    for i in range(runs):
        ev[2 * i].record()
        status = min(status, L.mla_prefill_run(*args))
        ev[2 * i + 1].record()
    binding.raise_for_status(status)
    torch.cuda.synchronize()
    st = stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) / 1e3 for i in range(runs)])
    rebuild = 2 * 2 * T * d_c * h * d_h                   # K and V from the latents
    attn = h * (T * (T + 1) // 2) * 2 * (d_h + d_r + d_h)  # causal scores over d_h + d_r, weighted values
    flops = rebuild + attn
    return dict(T=T, h=h, us={k: st[k] * 1e6 for k in ("mean", "median", "p10", "p90")}, runs=st["n"],
                algorithmic_flops=flops, rebuild_flops=rebuild, attention_flops=attn,
                roofline=dict(bound="mfma", achieved=flops / st["median"] / 1e12, peak=MFMA_BF16_TFLOPS,
                              unit="TFLOP/s", frac=flops / st["median"] / 1e12 / MFMA_BF16_TFLOPS,
                              what="median over the runs of one call (rebuild GEMM + attention)"))


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


def measured_counters(kernel, workload):
    """MFMA utilisation and LDS figures of one kernel from the committed
    rocprofv3 counter summary, or None when there is none or the kernel
    source changed since."""
    from mla_latent_cache_absorbed_amd.profiling import COUNTERS_FILE, source_digest
    try:
        with open(COUNTERS_FILE) as f:
            e = json.load(f)[kernel][workload]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("source_digest") != source_digest(kernel):
        return None
    return e


def host_cpu():
    """CPU model and core counts of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return dict(cpu_model=model, nproc=os.cpu_count(), usable_cpus=usable)


def oracle_rate(wl, target_s, threads=None):
    """TFLOP/s of the explicit fp64 oracle (as it stands) on a bounded sample
    of whole (sequence, head) pairs of the workload, sized for about target_s
    seconds; with `threads`, on that many OpenMP threads."""
    import oracle
    from mla_latent_cache_absorbed_amd import inputs
    prob = oracle.Problem(**inputs.oracle_problem_kwargs(wl))
    saved = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        used = oracle.num_threads()
        all_pairs = [(b, i) for b in range(wl.batch) for i in range(wl.h)]

        def run(n):
            pairs = all_pairs[:n]
            t = time.perf_counter()
            oracle.decode_explicit(prob, pairs)
            return time.perf_counter() - t, pairs

        n = min(len(all_pairs), max(1, used))
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
    finally:
        oracle.set_num_threads(saved)
    per_pair = 4 * wl.d_c + 2 * wl.d_r + 1
    flops = 0
    for b, _ in pairs:
        L = int(wl.lens[b])
        flops += sum(L - wl.n_q + m + 1 for m in range(wl.n_q)) * per_pair
        flops += wl.n_q * 2 * 2 * wl.d_h * wl.d_c
    return dict(value=flops / dt / 1e12, seconds=dt, reps=reps, pairs=len(pairs), of=len(all_pairs),
                threads=min(used, len(pairs)))


def cpu_baseline(wl, target_s=15.0):
    """The fp64 oracle (explicit K/V form, as it stands) timed on this host:
    on all its threads for the measured workload, and on one thread for the
    tiny fp32 and the T=4K configurations."""
    from mla_latent_cache_absorbed_amd import inputs
    main = oracle_rate(wl, target_s)
    one = {}
    for name in ("tiny_fp32", "ds2_t4k"):
        r = oracle_rate(inputs.make(name), 5.0, threads=1)
        one[name] = dict(value=r["value"], unit="TFLOP/s", seconds_per_pass=r["seconds"],
                         sample="%d of %d (sequence, head) pairs, mean of %d pass(es)"
                                % (r["pairs"], r["of"], r["reps"]))
    return dict(value=main["value"], unit="TFLOP/s", cores=main["threads"], kind="oracle",
                sample="explicit fp64 oracle (per-head K/V rebuilt, textbook softmax) on %d of "
                       "%d (sequence, head) pairs of %s, %.2f s wall per pass, mean of %d pass(es)"
                       % (main["pairs"], main["of"], wl.name, main["seconds"], main["reps"]),
                seconds=main["seconds"], one_thread=one, **host_cpu())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ds2_t32k",
                    help="headline workload (B=1, T=32K: the split kernel's roofline bar point)")
    ap.add_argument("--extra", default="ds2_t4k,ds2_t128k,ds2_paged_b32,ds2_mtp_b16",
                    help="comma-separated further workloads whose steps and kernels are also "
                         "measured ('' = none)")
    ap.add_argument("--dist-runs", type=int, default=100,
                    help="runs behind each median / p10 / p90 (at least --steps)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the copy and GEMM measurements of achievable peaks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-oproj", action="store_true", help="skip the output-projection measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="T",
                    help="only time prefill of a T-token prompt (for profiling) and print its record")
    ap.add_argument("--no-projections", action="store_true",
                    help="skip the cache-append and query-side measurements")
    ap.add_argument("--projections-only", type=int, default=0, metavar="ROWS",
                    help="only time the cache append and the query side of ROWS rows and print their records")
    ap.add_argument("--oproj-only", type=int, default=0, metavar="ROWS",
                    help="only time the output projection of ROWS rows (for profiling) and print its record")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the launch-floor runs (context lengths 1), e.g. under a profiler, "
                         "whose per-kernel averages would include them")
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

    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    dist_runs = max(args.dist_runs, args.steps)

    if args.oproj_only:
        print(json.dumps(measure_oproj(args.oproj_only, dist_runs, args.warmup)))
        return
    if args.prefill_only:
        print(json.dumps(measure_prefill(args.prefill_only, max(5, args.steps), args.warmup)))
        return
    if args.projections_only:
        print(json.dumps(measure_projections(args.projections_only, dist_runs, args.warmup)))
        return

    def measure(name, steps, warmup, with_floor=False):
        wl = inputs.make(name)
        dw = DeviceWorkload(wl)
        n_layers = args.layers or max(2, min(60, math.ceil(MIN_ROTATION_BYTES / layer_bytes(wl))))
        layers = Layers(dw, n_layers)
        splits, chunk = dw.split_plan()
        log("%s: %d layers rotated (%.0f MB each), %d chunks of %d tokens" %
            (name, n_layers, layer_bytes(wl) / 1e6, splits, chunk))
        step_s, _ = time_steps(dw, layers, steps, warmup, per_kernel=False)
        graph_s = None if args.no_graph else time_graph(dw, layers, steps, warmup)
        step_dist = stats(step_distribution(dw, layers, dist_runs))
        kern_dist = {k: stats(v) for k, v in kernel_distribution(dw, layers, dist_runs).items()}
        log("%s: step %.2f us (mean of %d); median %.2f us over %d; kernels (median us): %s" %
            (name, step_s * 1e6, steps, step_dist["median"] * 1e6, dist_runs,
             {k: round(v["median"] * 1e6, 2) for k, v in kern_dist.items()}))
        floor = None
        if with_floor:
            floor = {k: stats(v) for k, v in launch_floor(dw, layers, dist_runs).items()}
            log("%s: launch floor (context lengths 1), kernels (median us): %s" %
                (name, {k: round(v["median"] * 1e6, 2) for k, v in floor.items()}))
        c = counts(wl, chunk_count(wl, splits, chunk, num_cus))
        del layers
        return dict(wl=wl, c=c, step_s=step_s, graph_s=graph_s, step_dist=step_dist, kern=kern_dist,
                    splits=splits, chunk=chunk, n_layers=n_layers, floor=floor)

    def us(d):
        return {k: d[k] * 1e6 for k in ("mean", "median", "p10", "p90")}

    def roofline_of(m, kernel="split_attn"):
        wl, c, kd = m["wl"], m["c"], m["kern"][kernel]
        roof = kernel_roofline(kernel, c[kernel], kd["mean"], wl.dtype)
        roof["traffic"] = measured_traffic(kernel, wl.name)
        cnt = measured_counters(kernel, wl.name)
        roof["mfma_util"] = cnt.get("mfma_util") if cnt else None
        roof.update(kernel=kernel, workload=wl.name, avg_us=kd["mean"] * 1e6,
                    median_us=kd["median"] * 1e6, p10_us=kd["p10"] * 1e6, p90_us=kd["p90"] * 1e6,
                    runs=kd["n"])
        return roof

    def entry(m):
        wl, c = m["wl"], m["c"]
        t_split = m["kern"]["split_attn"]["mean"]
        return dict(
            step_us=m["step_s"] * 1e6, step_tflops=c["step"]["flops"] / m["step_s"] / 1e12,
            step_hbm_gbps=c["step"]["bytes"] / m["step_s"] / 1e9,
            graph_step_us=None if m["graph_s"] is None else m["graph_s"] * 1e6,
            step_dist_us=us(m["step_dist"]),
            kernels_us={k: us(v) for k, v in m["kern"].items()},
            splits=m["splits"], chunk_len=m["chunk"], layers_rotated=m["n_layers"],
            split_us=t_split * 1e6,
            cache_gbps=c["split_attn"]["bytes"] / t_split / 1e9,
            cache_plus_partials_gbps=(c["split_attn"]["bytes"] + c["split_attn"]["partial_bytes"])
            / t_split / 1e9,
            tflops=c["split_attn"]["flops"] / t_split / 1e12,
            roofline=roofline_of(m))

    head = measure(args.workload, args.steps, args.warmup, with_floor=not args.no_floor)
    wl, c = head["wl"], head["c"]
    rooflines = {k: kernel_roofline(k, c[k], v["mean"], wl.dtype) for k, v in head["kern"].items()}
    out = {
        "metric": METRIC,
        "value": c["step"]["flops"] / head["step_s"] / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_s"] * 1e3,
        "graph_ms_per_step": None if head["graph_s"] is None else head["graph_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q": wl.n_q,
                   "context": int(wl.max_len), "h": wl.h, "d_c": wl.d_c, "d_r": wl.d_r,
                   "d_h": wl.d_h, "page_size": wl.page_size, "splits": head["splits"],
                   "chunk_len": head["chunk"], "layers_rotated": head["n_layers"]},
        "cache_gbps": c["step"]["cache_bytes"] / head["step_s"] / 1e9,
        # the split kernel (scores, softmax and latent sums over the cache)
        # against its roofline at this workload
        "roofline": roofline_of(head),
        # the whole step against the same HBM peak: the bytes the method must
        # move per step (cache read once, W_UK and W_UV once) over its wall time
        "step_hbm": dict(algorithmic_bytes=c["step"]["bytes"], achieved=c["step"]["bytes"] / head["step_s"] / 1e9,
                         peak=HBM_GBPS, unit="GB/s",
                         frac=c["step"]["bytes"] / head["step_s"] / 1e9 / HBM_GBPS),
        "timing": dict(step_us=us(head["step_dist"]), runs=dist_runs,
                       how="per-step events on the launch stream; per-kernel start/stop events "
                           "recorded by each kernel's dispatch; mean/median/p10/p90 over the runs"),
        "kernels": {k: dict(us(head["kern"][k]), **rooflines[k]) for k in head["kern"]},
        # the same plan and grids with every context length 1 (the split
        # kernel's launch-and-drain floor at this grid)
        "launch_floor_us": None if head["floor"] is None else {k: us(v) for k, v in head["floor"].items()},
    }
    sweep = {}
    for name in [n for n in args.extra.split(",") if n]:
        m = measure(name, max(10, args.steps // 2), 5)
        sweep[name] = entry(m)
    if sweep:
        out["sweep"] = sweep

    if not args.no_oproj:
        # the next step after the decode path, measured on its own: the output
        # projection of the headline's rows and of the batched configurations'
        out["oproj"] = {"r%d" % r: measure_oproj(r, dist_runs, 10) for r in (1, 32, 64)}
        log("oproj (median us): %s" % {k: round(v["us"]["median"], 2) for k, v in out["oproj"].items()})
    if not args.no_prefill:
        # prefill of a 4K-token prompt (the T=4K decode configuration's context)
        out["prefill"] = {"t4k": measure_prefill(4096, 20, 3)}
        log("prefill T=4096 (median us): %.1f" % out["prefill"]["t4k"]["us"]["median"])
    if not args.no_projections:
        # the steps before the decode path, measured on their own: the cache
        # append and the query side of one and of 64 new tokens
        out["projections"] = {"r%d" % r: measure_projections(r, dist_runs, 10) for r in (1, 64)}
        log("projections (median us): %s" % {k: {kk: round(vv["us"]["median"], 2) for kk, vv in v.items()}
                                             for k, v in out["projections"].items()})

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
