#!/usr/bin/env python3
"""Decode throughput of grouped-query decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gqa_decode call: one new token for each of the B sequences of
the workload, attending over its seeded synthetic KV cache (inputs resident in
HBM before the timed region).  Prints ONE JSON line with tokens/s, the
roofline of the decode kernel (algorithmic bytes / average kernel time from
HIP events on the launch stream, against 8 TB/s), and the CPU oracle timed on
a bounded sample of the same workload.

Other modes (used to produce the files under profiles/):
    --variant append|window|layer   decode with the cache append, sliding-window
                               decode, the whole decode step of a layer
    --fig6                     the pages' fig. 6 group sweep as decoder attention
    --shapes                   serving shapes: batch 1..256, context 1K..128K
                               (one JSON line per shape)
    --meanpool                 the mean-pool conversion step (one JSON line)
    --calibrate-copy           plain device copy of a known size, for scaling
                               the FETCH_SIZE / WRITE_SIZE counters
    --read-ceiling             the streaming-read probe: what a kernel that only
                               reads (16-byte loads) gets from HBM
    --timeline                 per-phase timeline of matrix-core decode calls
                               (an instrumented build of the kernel)
    --summarize-rocprof DIR    print a summary of rocprofv3 CSV output
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "decode tokens/sec + achieved HBM GB/s (% of peak) for GQA decode at 1 GPU"
KERNEL_SOURCES = ["gqa_device.h", "gqa_decode_mfma.hip", "gqa_decode_mfma_f32.hip", "gqa_decode_valu.hip"]


def kernel_source_hash() -> str:
    """Hash of the decode kernels' code (comments and blank lines removed, so
    that editing documentation does not invalidate measured counters)."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "grouped_query_kv_decode_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [l.rstrip() for l in text.splitlines() if l.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def alg_bytes(w, seq_lens, variant: str = "decode", window: int = 0) -> int:
    """K+V bytes of the attended positions plus q and out (element bytes e);
    with a window only the last `window` positions count; the cache append
    adds the new rows written into the cache (their reads replace cache reads)."""
    e = 4 if w.dtype == "f32" else 2
    lens = seq_lens.to("cpu").clamp(0, w.Lmax)
    if window > 0:
        lens = lens.clamp(max=window)
    n = int(lens.sum())
    kv = 2 * w.G * n * w.d * e
    if variant == "layer":
        # weights read once; x read, q/key/val and the attention output written
        # and read back, y written; the cache rows of the new token written
        dm, nqkv = w.d_model, (w.H + 2 * w.G) * w.d
        weights = (dm * nqkv + w.H * w.d * dm) * e
        acts = w.B * (dm + 2 * nqkv + 2 * w.H * w.d + dm) * e
        return kv + weights + acts + 2 * w.B * w.G * w.d * e
    extra = 2 * w.B * w.G * w.d * e if variant == "append" else 0
    return kv + 2 * w.B * w.H * w.d * e + extra


def load_traffic(workload_name: str):
    """HBM traffic per dispatch from committed counter runs, if they were taken
    on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_dispatch")


# The pages' only timing figures: T5-XXL inference time per sample (whole
# encoder-decoder model, averaged over the paper's tasks, on hardware the
# pages do not name) - context for the decode rates, not a target
# (wikillm "Grouped-query attention (GQA)", When to use which; elemedex
# glossary "grouped-query attention", paragraph "Grouped (GQA)").
PAGES_T5XXL_SECONDS_PER_SAMPLE = {"MHA": 1.51, "GQA-8": 0.28, "MQA": 0.24}


def host_threads():
    """(threads, affinity cores, reason): the oracle takes every core of this
    process's affinity mask, or OMP_NUM_THREADS when the launcher sets it
    lower (a GPU host's per-GPU share of its cores)."""
    aff = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    cap = int(omp) if omp.isdigit() and int(omp) > 0 else 0
    if cap and cap < aff:
        return cap, aff, "OMP_NUM_THREADS=%d, the host's share of its %d affinity cores for this GPU" % (cap, aff)
    return aff, aff, "every core of the affinity mask"


def versions():
    import torch
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"torch": torch.__version__, "hip_runtime": torch.version.hip, "rocm": rocm,
            "python": sys.version.split()[0]}


def cpu_baseline(w, q, k, v, lens, out_gpu, budget_s: float):
    """Times the oracle on the host cores over whole batches of the workload."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import oracle
    threads, aff, why = host_threads()
    # host copies of the attended part of the cache, one sequence at a time
    t_copy = time.perf_counter()
    seqs = []
    for b in range(w.B):
        n = max(1, min(int(lens[b]), w.Lmax))
        seqs.append((q[b:b + 1].cpu(), k[b:b + 1, :, :n].cpu().contiguous(), v[b:b + 1, :, :n].cpu().contiguous(),
                     lens[b:b + 1].cpu()))
    t_copy = time.perf_counter() - t_copy
    ora = oracle.get()
    reps, elapsed, ref = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        outs = [ora.decode(qq, kk, vv, ll, w.scale, nthreads=threads)[0] for qq, kk, vv, ll in seqs]
        elapsed += time.perf_counter() - t0
        reps += 1
        if ref is None:
            ref = np.stack(outs)
        if elapsed >= budget_s or reps >= 100000:
            break
    # single-thread reference: one sequence of the batch, scaled to the batch
    qq, kk, vv, ll = seqs[0]
    t0 = time.perf_counter()
    ora.decode(qq, kk, vv, ll, w.scale, nthreads=1)
    t_one = time.perf_counter() - t0
    got = out_gpu.float().cpu().double().numpy()
    err = float(np.max(np.abs(got - ref)))
    tol = 1e-5 if w.dtype == "f32" else 2e-2
    base = {
        "value": w.B * reps / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": "%d full batch(es) of the workload (%d sequences each), binary64 C oracle, %d threads over "
                  "(sequence, head); host copy %.2f s excluded" % (reps, w.B, threads, t_copy),
        "threads_reason": why, "affinity_cores": aff, "host_cpu_count": os.cpu_count(),
        "seconds_per_batch": elapsed / reps,
        # one sequence on one thread, scaled to the batch (uniform lengths only)
        "single_thread_seconds_per_batch": t_one * w.B if not w.ragged else None,
    }
    parity = {"max_abs_err": err, "tol": tol, "pass": bool(err <= tol and np.isfinite(got).all())}
    return base, parity


def run_bench(args):
    import torch
    import grouped_query_kv_decode_amd as gqa
    from grouped_query_kv_decode_amd import workloads as wl

    if args.shape:
        # an unnamed shape (kernel comparisons, plan checks): full-length
        # caches, N(0,1) values, seed 5
        B, H, G, d, L = (int(x) for x in args.shape.split(","))
        dt = args.dtype or "bf16"
        w = wl.Workload("shape_%s_B%d_H%d_G%d_d%d_L%d" % (dt, B, H, G, d, L), B, H, G, d, L, dt, 5)
    else:
        w = wl.WORKLOADS[args.workload]
    if args.dtype == "f32" and args.variant == "layer":
        raise SystemExit("--variant layer runs the bf16 projections: use --dtype bf16")
    if args.dtype and args.dtype != w.dtype:
        # the same shape and seeds in the other storage type (binary32 runs on
        # the VALU kernel); the name says which
        w = w.with_(dtype=args.dtype, name=w.name.replace("_" + w.dtype + "_", "_" + args.dtype + "_"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gqa.load_library()
    kv_bytes = 2 * w.B * w.G * w.Lmax * w.d * (4 if w.dtype == "f32" else 2)
    rot = args.rotate if args.rotate else max(1, math.ceil((1 << 30) / kv_bytes))
    window = args.window if args.variant in ("window", "append") else 0
    # --graph: the calls are bound to a side stream and the K timed steps are
    # captured there into one HIP graph, replayed once in the timed region
    # (what a serving loop replaying graphs sees: no host launch cost).
    side = torch.cuda.Stream(dev) if args.graph else None
    if side is not None:
        torch.cuda.set_stream(side)
    sets, decs = [], []
    for i in range(rot):
        q, k, v, lens = wl.make_inputs(w, dev, pad="none", seed_offset=i)
        if args.variant == "layer":
            gen = torch.Generator(dev).manual_seed(w.seed + 7 * i)
            dm, nqkv = w.d_model, (w.H + 2 * w.G) * w.d
            x = torch.randn((w.B, dm), generator=gen, device=dev).to(k.dtype)
            w_qkv = (torch.randn((dm, nqkv), generator=gen, device=dev) * dm ** -0.5).to(k.dtype)
            w_o = (torch.randn((w.H * w.d, dm), generator=gen, device=dev) * (w.H * w.d) ** -0.5).to(k.dtype)
            dec = gqa.LayerStep(x, w_qkv, w_o, k, v, lens, w.H, w.G, w.scale)
        elif args.variant == "append":
            gen = torch.Generator(dev).manual_seed(w.seed + 7 * i)
            kn = torch.randn((w.B, w.G, w.d), generator=gen, device=dev).to(k.dtype)
            vn = torch.randn((w.B, w.G, w.d), generator=gen, device=dev).to(k.dtype)
            dec = gqa.Decoder(q, k, v, lens, w.scale, window=window, k_new=kn, v_new=vn)
        else:
            dec = gqa.Decoder(q, k, v, lens, w.scale, window=window)
        sets.append((q, k, v, lens))
        decs.append(dec)
    torch.cuda.synchronize()
    kind = gqa.decode_kernel_kind(w.B, w.H, w.G, w.d, w.Lmax, gqa.GQA_F32 if w.dtype == "f32" else gqa.GQA_BF16)

    for i in range(args.warmup):
        decs[i % rot]()
    torch.cuda.synchronize()

    # A step is one gqa_decode call.  Two HIP events on the launch stream
    # bracket the timed region; with one kernel per call their difference / K
    # is the kernel's average duration including the back-to-back launch gaps.
    K = args.steps
    stream = torch.cuda.current_stream()
    graph = None
    if side is not None:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(K):
                decs[i % rot]()
        graph.replay()
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            decs[i % rot]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_kernel_ms = ev0.elapsed_time(ev1) / K
    code = gqa.GQA_F32 if w.dtype == "f32" else gqa.GQA_BF16
    split = gqa.decode_workspace_size(w.B, w.H, w.G, w.d, w.Lmax, code) > 0
    kernels_per_step = 2 if split and os.environ.get("GQA_MERGE") == "kernel" else 1
    if args.variant == "layer":
        kernels_per_step += 2
    ab = alg_bytes(w, sets[0][3], args.variant, window)  # every rotation set has the same lengths
    achieved = ab / (avg_kernel_ms * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / K
    traffic = load_traffic(w.name) if args.variant == "decode" else None

    line = {
        "metric": METRIC,
        "value": w.B * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian caches)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "G": w.G, "d": w.d, "Lmax": w.Lmax,
                   "ragged": w.ragged, "rotation_sets": rot, "variant": args.variant, "window": window,
                   "kernel": ["valu", "mfma"][kind], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic},
        "alg_bytes_per_step": ab,
        "kernel_us_avg": avg_kernel_ms * 1e3,
        "timing": "hip_graph" if graph is not None else "eager",
        "kernels_per_step": kernels_per_step,
        "hbm_gbps_wall": ab / (ms_per_step * 1e-3) / 1e9,
        # counter traffic (FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a
        # plain copy's counts) over the kernel time, and against the
        # algorithmic bytes; null when the counters predate the kernel sources
        "fetch_GBps": traffic / (avg_kernel_ms * 1e-3) / 1e9 if traffic else None,
        "over_fetch_ratio": traffic / ab if traffic else None,
        "seed": w.seed,
        "versions": versions(),
        "context": {"pages_t5xxl_seconds_per_sample": PAGES_T5XXL_SECONDS_PER_SAMPLE,
                    "note": "whole-model T5-XXL inference time per sample on unnamed hardware (the pages' only "
                            "timings); not comparable with one attention layer's decode call"},
    }
    if not args.no_cpu_baseline and args.variant == "decode":
        q, k, v, lens = sets[0]
        out = decs[0]().clone()
        torch.cuda.synchronize()
        base, parity = cpu_baseline(w, q, k, v, lens.cpu(), out, args.cpu_budget)
        line["cpu_baseline"] = base
        line["parity"] = parity
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def fig6(args):
    """The group sweep of the pages' Fig. 6 setup (input 2048, output 512) as
    decoder attention on one GPU, per layer: for each of 512 output steps, a
    self-attention decode with the cache append over the growing decoder cache
    (lengths 1 .. 512) and a cross-attention decode over the 2048 encoder
    positions.  T5-XXL shape: H = 64 heads of d = 64; G swept; B sequences.
    Prints one JSON line per G (GPU time from HIP events on the launch stream)."""
    import torch
    import grouped_query_kv_decode_amd as gqa
    from grouped_query_kv_decode_amd import workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, d, T_in, T_out = args.fig6_batch, 64, 64, 2048, 512
    for G in wl.T5XXL_SWEEP_G:
        self_w = wl.Workload("fig6_self_G%d" % G, B, H, G, d, T_out, "bf16", 2000 + G, value_scale=0.5)
        cross_w = wl.Workload("fig6_cross_G%d" % G, B, H, G, d, T_in, "bf16", 3000 + G, value_scale=0.5)
        q, ks, vs, _ = wl.make_inputs(self_w, dev, pad="zero", seq_lens=torch.zeros(B, dtype=torch.int32))
        _, kx, vx, lx = wl.make_inputs(cross_w, dev, pad="none")
        gen = torch.Generator(dev).manual_seed(4000 + G)
        k_new = (torch.randn((T_out, B, G, d), generator=gen, device=dev) * 0.5).to(torch.bfloat16)
        v_new = (torch.randn((T_out, B, G, d), generator=gen, device=dev) * 0.5).to(torch.bfloat16)
        lens = [torch.full((B,), t + 1, dtype=torch.int32, device=dev) for t in range(T_out)]
        self_dec = [gqa.Decoder(q, ks, vs, lens[t], self_w.scale, k_new=k_new[t], v_new=v_new[t])
                    for t in range(T_out)]
        cross_dec = gqa.Decoder(q, kx, vx, lx, cross_w.scale)
        for t in range(8):
            self_dec[t]()
            cross_dec()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for t in range(T_out):
            self_dec[t]()
            cross_dec()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_s = e0.elapsed_time(e1) * 1e-3
        e = 2
        self_bytes = sum(2 * G * (t + 1) * d * e for t in range(T_out)) * B + T_out * 2 * B * G * d * e
        cross_bytes = T_out * 2 * G * T_in * d * e * B
        qo_bytes = T_out * 2 * (2 * B * H * d * e)
        ab = self_bytes + cross_bytes + qo_bytes
        print(json.dumps({
            "mode": "fig6", "G": G, "B": B, "H": H, "d": d, "input_len": T_in, "output_len": T_out,
            "gpu_s_per_layer": gpu_s, "wall_s_per_layer": wall, "ms_per_output_step": gpu_s * 1e3 / T_out,
            "tokens_per_s": B * T_out / gpu_s, "alg_GBps": ab / gpu_s / 1e9, "frac_of_8TBps": ab / gpu_s / 8e12,
            "note": "attention only, one decoder layer; the pages' fig. 6 times whole T5-XXL inference per sample",
        }), flush=True)
        del q, ks, vs, kx, vx, k_new, v_new, self_dec, cross_dec
        torch.cuda.empty_cache()


def read_ceiling(args):
    """The practical HBM read ceiling: gqa_stream_read over 1 GiB buffers (4,
    rotated: beyond the 256 MB Infinity Cache), plain and non-temporal 16-byte
    loads, several grid sizes.  One JSON line per setting, then the best."""
    import torch
    import grouped_query_kv_decode_amd as gqa
    dev = torch.device("cuda:0")
    gqa.load_library()
    n = 1 << 30
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(4)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    best = None
    for nt in (False, True):
        for grid in (1024, 2048, 4096, 8192):
            for i in range(3):
                gqa.stream_read(bufs[i % 4], nt, grid, sink)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            iters = 40
            e0.record(stream)
            for i in range(iters):
                gqa.stream_read(bufs[i % 4], nt, grid, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / iters
            line = {"mode": "read_ceiling", "nontemporal": nt, "grid": grid, "bytes": n, "us_per_call": us,
                    "GBps": n / us / 1e3, "frac_of_8TBps": n / us / 8e6}
            print(json.dumps(line), flush=True)
            if best is None or line["GBps"] > best["GBps"]:
                best = line
    print(json.dumps(dict(best, mode="read_ceiling_best")), flush=True)
    # The floor of a call: the same kernel reading one 16-byte piece, on 1 and
    # on 256 workgroups, 400 calls back to back from this Python loop (bound
    # by the host's cost per call) and as one replay of a HIP graph of the
    # 400 calls (the GPU's own cost per launch).
    tiny = bufs[0][:16]
    iters = 400
    for grid in (1, 256):
        for i in range(20):
            gqa.stream_read(tiny, True, grid, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            gqa.stream_read(tiny, True, grid, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) * 1e3 / iters
        side = torch.cuda.Stream(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(iters):
                gqa.stream_read(tiny, True, grid, sink)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "launch_floor", "grid": grid, "bytes": 16, "us_per_call": eager,
                          "us_per_call_graph": e0.elapsed_time(e1) * 1e3 / iters}), flush=True)


def calibrate_copy(args):
    """A plain device-to-device copy of a known size (for counter scaling)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "calls": args.steps}), flush=True)


def meanpool_bench(args):
    """The conversion step (mean-pool of the K or V projection within each
    group) on the Mistral-7B shapes: W [4096, 32*128] binary32 -> [4096, 8*128].
    One JSON line: time per call and algorithmic bytes (read W once, write the
    result once) / time against 8 TB/s.  (Bit-exactness against the oracle is
    checked by the GPU tests.)"""
    import torch
    import grouped_query_kv_decode_amd as gqa
    dev = torch.device("cuda:0")
    d_model, H, G, h = 4096, 32, 8, 128
    gen = torch.Generator(dev).manual_seed(1234)
    rot = 8  # 8 x 64 MiB inputs: beyond the 256 MB Infinity Cache
    ws = [torch.randn((d_model, H * h), generator=gen, device=dev) for _ in range(rot)]
    out = torch.empty((d_model, G * h), dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        gqa.meanpool_kv(ws[i % rot], H, G, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        gqa.meanpool_kv(ws[i % rot], H, G, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    ab = d_model * H * h * 4 + d_model * G * h * 4
    print(json.dumps({"mode": "meanpool", "d_model": d_model, "H": H, "G": G, "h": h, "dtype": "f32",
                      "us_per_call": us, "alg_bytes": ab, "alg_GBps": ab / us / 1e3,
                      "frac_of_8TBps": ab / us / 8e6, "steps": args.steps}), flush=True)


# Serving shapes beyond the named workloads (bfloat16, full-length caches):
# (H, G, d) of common models - 32/8/128 Llama-3-8B-like, 8/1/128 one GPU's
# share of a 64-query-head, 8-K/V-head model split 8 ways, 32/16/128 Gemma-2-
# like, 64/4/128 a wide group, 16/8/64 - at batch 1 .. 256, contexts 1K .. 128K.
SERVING_HEADS = [(32, 8, 128), (8, 1, 128), (32, 16, 128), (64, 4, 128), (16, 8, 64)]
SERVING_BL = [(1, 1024), (1, 32768), (1, 131072), (3, 8192), (4, 8192), (12, 4096), (16, 1024), (20, 4096),
              (48, 2048), (64, 2048), (64, 8192), (256, 1024), (256, 4096)]


def shapes_bench(args):
    """One JSON line per serving shape: time per gqa_decode call (HIP events
    over back-to-back calls, inputs rotated through >= 1 GiB where memory
    allows) and algorithmic bytes / time against 8 TB/s (bf16, or the
    dtype given)."""
    import torch
    import grouped_query_kv_decode_amd as gqa
    from grouped_query_kv_decode_amd import workloads as wl
    dev = torch.device("cuda:0")
    gqa.load_library()
    stream = torch.cuda.current_stream()
    dtype = args.dtype or "bf16"
    e = 4 if dtype == "f32" else 2
    code = gqa.GQA_F32 if dtype == "f32" else gqa.GQA_BF16
    for (H, G, d) in SERVING_HEADS:
        for (B, L) in SERVING_BL:
            kvb = 2 * B * G * L * d * e
            if kvb > (8 << 30):
                continue
            w = wl.Workload("serving_B%d_H%d_G%d_d%d_L%d" % (B, H, G, d, L), B, H, G, d, L, dtype, 5)
            rot = min(16, max(2, (1 << 30) // kvb))
            sets = [wl.make_inputs(w, dev, pad="none", seed_offset=i) for i in range(rot)]
            decs = [gqa.Decoder(q, k, v, lens, w.scale) for (q, k, v, lens) in sets]
            ab = kvb + 2 * B * H * d * e
            for i in range(10):
                decs[i % rot]()
            n = max(20, min(400, int(2e5 / max(1.0, ab / 7e6))))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n):
                decs[i % rot]()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            kind = gqa.decode_kernel_kind(B, H, G, d, L, code)
            splits = gqa.decode_workspace_size(B, H, G, d, L, code) > 0
            print(json.dumps({"mode": "shapes", "B": B, "H": H, "G": G, "d": d, "Lmax": L, "dtype": dtype,
                              "kernel": ["valu", "mfma"][kind], "split": splits, "steps": n, "rotation_sets": rot,
                              "us_per_call": us, "alg_bytes": ab, "alg_GBps": ab / us / 1e3,
                              "frac_of_8TBps": ab / us / 8e6}), flush=True)
            del sets, decs
            torch.cuda.empty_cache()


def counter_mean(d, counter, kernel_substr):
    """Mean per-dispatch value of a rocprofv3 --pmc counter for kernels whose name contains kernel_substr."""
    vals = [float(r["Counter_Value"]) for r in _read_csvs(d, "counter_collection.csv")
            if r.get("Counter_Name") == counter and kernel_substr in r.get("Kernel_Name", "")]
    vals += [v for (k, c, v) in _db_rows(d)[1] if c == counter and kernel_substr in k]
    if not vals:
        raise SystemExit("no %s samples for %s in %s" % (counter, kernel_substr, d))
    return sum(vals) / len(vals), len(vals)


def write_traffic(args):
    """HBM bytes per dispatch of the decode kernel from FETCH_SIZE / WRITE_SIZE
    passes (KiB per dispatch), each scaled by what the same counter reads for a
    plain 1 GiB device copy; written to profiles/traffic_<workload>.json."""
    fetch, nf = counter_mean(args.fetch_dir, "FETCH_SIZE", "decode_")
    write, nw = counter_mean(args.write_dir, "WRITE_SIZE", "decode_")
    cf, _ = counter_mean(args.copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _ = counter_mean(args.copy_write_dir, "WRITE_SIZE", "copyBuffer")
    copy_kib = (1 << 30) / 1024.0
    f_fac, w_fac = cf / copy_kib, cw / copy_kib
    rec = {
        "workload": args.workload, "source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write, "dispatches": [nf, nw],
        "copy_fetch_factor": f_fac, "copy_write_factor": w_fac,
        "bytes_per_dispatch": (fetch / f_fac + write / w_fac) * 1024.0,
    }
    path = os.path.join(args.traffic_dir or os.path.join(ROOT, "profiles"), "traffic_%s.json" % args.workload)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _read_csvs(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _db_rows(d):
    """(kernel durations, counter samples) from rocprofv3's SQLite output
    (*_results.db, its default format): {name: [ns, ...]}, [(kernel, counter, value)]."""
    import sqlite3
    durs, ctr = {}, []
    for f in sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)):
        con = sqlite3.connect(f)
        for name, dur in con.execute("select name, end - start from kernels"):
            durs.setdefault(name, []).append(float(dur))
        for kname, cname, val in con.execute("select kernel_name, counter_name, value from counters_collection"):
            ctr.append((kname, cname, float(val)))
        con.close()
    return durs, ctr


def summarize_rocprof(d):
    """Per-kernel duration stats and per-dispatch counter means from rocprofv3
    output (CSV files or the SQLite database)."""
    stats = _read_csvs(d, "kernel_stats.csv")
    out = []
    durs, dbctr = _db_rows(d)
    if durs:
        out.append("kernel stats (rocprofv3 --kernel-trace, from the results database):")
        out.append("%-90s %7s %10s %10s %10s %10s" % ("kernel", "calls", "avg_us", "median_us", "min_us", "max_us"))
        for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            v = sorted(v)
            out.append("%-90s %7d %10.2f %10.2f %10.2f %10.2f" % (name[:90], len(v), sum(v) / len(v) / 1e3,
                                                               v[len(v) // 2] / 1e3, v[0] / 1e3, v[-1] / 1e3))
    if dbctr:
        agg = {}
        for kname, cname, val in dbctr:
            agg.setdefault((kname, cname), []).append(val)
        out.append("counters (rocprofv3 --pmc), mean per dispatch:")
        for (kname, cname), vals in sorted(agg.items()):
            out.append("%-90s %-12s n=%-5d mean=%.1f" % (kname[:90], cname, len(vals), sum(vals) / len(vals)))
    if stats:
        out.append("kernel stats (rocprofv3 --kernel-trace --stats):")
        out.append("%-90s %7s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
        for r in stats:
            out.append("%-90s %7s %12.2f %12.2f %12.2f" % (r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                          float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    ctr = _read_csvs(d, "counter_collection.csv")
    if ctr:
        agg = {}
        for r in ctr:
            key = (r.get("Kernel_Name", "?"), r.get("Counter_Name", "?"))
            agg.setdefault(key, []).append(float(r.get("Counter_Value", "nan")))
        out.append("counters (rocprofv3 --pmc), mean per dispatch:")
        for (kname, cname), vals in sorted(agg.items()):
            out.append("%-90s %-12s n=%-5d mean=%.1f" % (kname[:90], cname, len(vals), sum(vals) / len(vals)))
    return "\n".join(out)


# the per-phase timeline: the bench default, the small calls, and the largest T5-XXL
# point that needs no split (workload, window)
TIMELINE_CASES = [("tiny_f32_B1_H8_G2_d64_L256", 0),
                  ("mistral7b_bf16_B16_H32_G8_d128_L4096", 0), ("t5xxl_bf16_B32_H64_G1_d64_L2048", 0),
                  ("t5xxl_bf16_B32_H64_G4_d64_L2048", 0), ("t5xxl_bf16_B32_H64_G8_d64_L2048", 0),
                  ("mistral7b_bf16_B16_H32_G8_d128_L4096", 1024)]

ALL_WORKLOADS = ["tiny_f32_B1_H8_G2_d64_L256", "mistral7b_bf16_B16_H32_G8_d128_L4096",
                 "t5xxl_bf16_B32_H64_G1_d64_L2048", "t5xxl_bf16_B32_H64_G4_d64_L2048",
                 "t5xxl_bf16_B32_H64_G8_d64_L2048", "t5xxl_bf16_B32_H64_G16_d64_L2048",
                 "t5xxl_bf16_B32_H64_G64_d64_L2048", "gemma2_27b_bf16_B8_H32_G16_d128_L8192",
                 "ragged_bf16_B64_H64_G8_d128_Lmax32768"]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mistral7b_bf16_B16_H32_G8_d128_L4096",
                    help="a named workload, or 'all' (one JSON line per named workload)")
    ap.add_argument("--shape", metavar="B,H,G,d,L", help="an unnamed full-length shape instead of a workload")
    ap.add_argument("--rotate", type=int, default=0, help="input sets cycled through (default: >= 1 GiB of caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", choices=["bf16", "f32"], default=None,
                    help="storage type of q, caches and output (default: the workload's)")
    ap.add_argument("--graph", action="store_true",
                    help="time one replay of the K steps captured into a HIP graph (no host launch cost)")
    ap.add_argument("--variant", choices=["decode", "append", "window", "layer"], default="decode",
                    help="decode (default), decode with the cache append, sliding-window decode, or the whole "
                         "decode step of a layer (q/k/v projection, append + attention, output projection)")
    ap.add_argument("--window", type=int, default=4096, help="window for --variant window/append (0: none)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time to aim for")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--read-ceiling", action="store_true", help="the streaming-read probe (read ceiling of HBM)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-phase timeline of matrix-core decode calls (needs libgqa_timeline.so: "
                         "python -m grouped_query_kv_decode_amd.timeline build)")
    ap.add_argument("--meanpool", action="store_true", help="time the K/V mean-pool conversion step")
    ap.add_argument("--fig6", action="store_true", help="the pages' fig. 6 group sweep as decoder attention")
    ap.add_argument("--fig6-batch", type=int, default=32)
    ap.add_argument("--shapes", action="store_true", help="serving shapes sweep (batch 1..256, context 1K..128K)")
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--write-traffic", action="store_true",
                    help="combine counter runs (--fetch-dir, --write-dir, --copy-fetch-dir, --copy-write-dir)")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--traffic-dir", help="where --write-traffic puts traffic_<workload>.json (default profiles/)")
    args = ap.parse_args()
    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof))
        return 0
    if args.write_traffic:
        write_traffic(args)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (collectives and sharding are out of "
              "scope); run with --gpus 1", file=sys.stderr)
        return 2
    if args.meanpool:
        meanpool_bench(args)
        return 0
    if args.calibrate_copy:
        calibrate_copy(args)
        return 0
    if args.read_ceiling:
        read_ceiling(args)
        return 0
    if args.timeline:
        from grouped_query_kv_decode_amd import timeline
        timeline.run(TIMELINE_CASES)
        return 0
    if args.fig6:
        fig6(args)
        return 0
    if args.shapes:
        shapes_bench(args)
        return 0
    if args.workload == "all":
        # every named workload, one JSON line each (the T5-XXL shape at every group count)
        import gc
        import torch
        from grouped_query_kv_decode_amd import workloads as wl
        for name in ALL_WORKLOADS:
            args.workload = name
            run_bench(args)
            gc.collect()
            torch.cuda.empty_cache()
        return 0
    run_bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
