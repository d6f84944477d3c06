#!/usr/bin/env python3
"""MLA latent-KV decode benchmark on one MI355X.

A step is one decode step of the whole model's attention: for each of the
40 layers, the hot path runs once over the batch's new query tokens: YaRN
RoPE of their query and key rope parts, append of their cache rows,
absorption of W_UK into the query, split-KV flash decoding over the latent
cache, LSE combine and the W_UV up-projection.  Every layer has its own
cache and kv_b_proj weights, all resident in HBM before timing starts.

Default workload: batch 1, one query token, context 32768, contiguous cache
(the 32K configuration of the headline metric).  The 256K configuration
(context 262144, KV chunks of 4096 and the device-balanced split) is
reported alongside under "ctx256k", and the 32K and 256K workloads over the
8-bit latent cache (E4M3 codes with per-128 fp32 scales, 656 bytes per token
and layer) under "fp8_cache".  "other_workloads" reports the batched paged
decode (16 x 65536), speculative verify of 2, 3 and 4 query tokens per
sequence (batch 32, log-uniform contexts in [4096, 131072], paged), verify
of 2 tokens over the 8-bit cache, and one sequence of 524288 tokens, all
with the device-balanced split; "prefill" the
chunked prefill (un-absorbed form) of 4096 new tokens on 32K and 128K
contexts, in TFLOP/s against the 2.5 PFLOP/s bf16 matrix peak.
"ctx1k_one_layer" times one decode call on a 1024-token context (one layer)
hot and after a 512 MiB write that flushes the caches; "read_ceiling" is
the best rate of the library's streaming-read probe over 1 and 4 GiB, the
practical HBM read ceiling on the same device; "kernel_tflops" fields are
algorithmic flops (69,632 per visible token and query token) over the
split-KV kernel's duration.  "cpu_baseline" also carries the absorbed fp64
CPU reference timed on the same layers.

Output: one JSON line.  "value" is decode tokens/s (batch * query tokens per
step / step time, timed over --steps replays of a HIP graph of the step).
"roofline" covers the split-KV kernel: algorithmic latent bytes per launch
(1152 B per visible cached token) over its average duration, measured with
HIP events that the kernel dispatches record themselves (hipExtLaunchKernel)
on the stream they run on; "traffic" is the HBM bytes per launch from the
committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters of the same kernel
source on the same workload, scaled by a calibration copy (else null).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + latent-KV GB/s (% HBM peak) at 32K and 256K ctx, 1 GPU"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak, 2.5 PFLOP/s
FLOPS_PER_TOKEN_QUERY = 2 * 32 * 576 + 2 * 32 * 512   # scores + value product per (visible token, query token)
BYTES_PER_TOKEN_LAYER = 1152    # 576 bf16 cached values per token per layer
BYTES_PER_TOKEN_LAYER_FP8 = 656  # 512 E4M3 codes + 4 fp32 scales + 64 bf16 rope values
COUNTERS = os.path.join(ROOT, "profiles", "splitkv_decode_counters.json")
DECODE_SRC = [os.path.join(ROOT, "mla_latent_kv_absorbed_amd", "csrc", f) for f in ("decode.hip", "mla_internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the split-KV kernel's sources (the kernel file and the shared definitions) with
    comments and whitespace runs removed: an edit of the code invalidates a counter record, an
    edit of a comment does not."""
    import re

    h = hashlib.sha256()
    for path in DECODE_SRC:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def run_workload(k: int, steps: int, warmup: int, use_graph: bool, kv_chunk=None, label="", cache_dtype="bf16"):
    import torch
    import mla_latent_kv_absorbed_amd as M
    from mla_latent_kv_absorbed_amd.workload import DeviceWorkload
    from synth.configs import workload

    wl = workload(k)
    dw = DeviceWorkload(wl, kv_chunk=kv_chunk, cache_dtype=cache_dtype)
    t0 = time.perf_counter()
    layers = [dw.build_layer(l) for l in range(wl.layers)]
    torch.cuda.synchronize()
    log(f"[{label}] built {wl.layers} layers of {wl.name} in {time.perf_counter() - t0:.1f}s "
        f"(chunk {dw.chunk_used}, {'paged' if dw.paged else 'contiguous'})")
    B, Sq = dw.B, dw.Sq
    outs = [torch.empty((B, Sq, 32, 128), dtype=torch.bfloat16, device=dw.dev) for _ in layers]
    lses = [torch.empty((B, Sq, 32), dtype=torch.float32, device=dw.dev) for _ in layers]

    def step():
        for li, o, l in zip(layers, outs, lses):
            dw.step(li, out=o, lse=l)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    graph = None
    if use_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            for _ in range(3):
                graph.replay()
                torch.cuda.synchronize()
                if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
                    raise RuntimeError("graph replay differs from eager step")
        except Exception as e:  # noqa: BLE001
            log(f"[{label}] graph capture unavailable ({e}); timing eager launches")
            graph = None

    run = graph.replay if graph is not None else step
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
        raise RuntimeError("timed steps changed the result")

    # split-KV kernel durations: HIP events recorded by the library around
    # the kernel, on the stream it is launched on, over `steps` eager steps
    M.mla_timing_enable(steps * len(layers))
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern_ms, launches = M.mla_timing_collect()
    M.mla_timing_disable()

    tokens_ctx = sum(dw.lens)
    bytes_per_launch = tokens_ctx * (BYTES_PER_TOKEN_LAYER_FP8 if cache_dtype == "fp8" else BYTES_PER_TOKEN_LAYER)
    avg_kernel_s = kern_ms / 1e3 / launches
    # query token j of sequence b sees L_b - Sq + j + 1 tokens
    visible = sum(L * Sq - Sq * (Sq - 1) // 2 for L in dw.lens)
    flops_per_launch = FLOPS_PER_TOKEN_QUERY * visible
    step_bytes = bytes_per_launch * len(layers)
    res = dict(
        workload=wl.name, batch=B, query_tokens=Sq, context=list(dw.lens) if B <= 4 else f"{B} seqs, sum {tokens_ctx}",
        layers=len(layers), layout="paged" if dw.paged else "contiguous", kv_chunk=dw.chunk_used,
        cache_dtype=cache_dtype,
        graph=graph is not None, ms_per_step=ms_per_step, tokens_per_s=B * Sq / (ms_per_step / 1e3),
        step_latent_gbps=step_bytes / (ms_per_step / 1e3) / 1e9,
        kernel_avg_us=avg_kernel_s * 1e6, kernel_bytes_per_launch=bytes_per_launch,
        kernel_latent_gbps=bytes_per_launch / avg_kernel_s / 1e9,
        kernel_tflops=flops_per_launch / avg_kernel_s / 1e12,
    )
    del layers, outs, lses, ref, graph
    torch.cuda.empty_cache()
    return res


def run_latency(k: int, kv_chunk: int, reps: int = 50, flush_mb: int = 512):
    """One decode call of the one-layer workload k, in a HIP graph: microseconds per call hot
    (200 back-to-back replays) and cold (median over `reps` replays, each after a
    flush_mb MiB write that evicts the 256 MB Infinity Cache and the L2s)."""
    import statistics
    import torch
    from mla_latent_kv_absorbed_amd.workload import DeviceWorkload
    from synth.configs import workload

    wl = workload(k)
    dw = DeviceWorkload(wl, kv_chunk=kv_chunk)
    li = dw.build_layer(0)
    out = torch.empty((dw.B, dw.Sq, 32, 128), dtype=torch.bfloat16, device=dw.dev)
    lse = torch.empty((dw.B, dw.Sq, 32), dtype=torch.float32, device=dw.dev)
    dw.step(li, out=out, lse=lse)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.step(li, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.step(li, out=out, lse=lse)
    for _ in range(5):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(200):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    hot_us = a.elapsed_time(b) / 200 * 1e3
    scratch = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dw.dev)
    cold = []
    for r in range(reps):
        scratch.fill_(r & 255)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b) * 1e3)
    res = dict(workload=wl.name, context=list(dw.lens), kv_chunk=dw.chunk_used, hot_us_per_call=hot_us,
               cold_us_per_call=statistics.median(cold), flush_mb=flush_mb)
    del li, dw, out, lse, graph, scratch
    torch.cuda.empty_cache()
    return res


def read_ceiling(sizes=(1 << 30, 4 << 30), reps: int = 10):
    """GB/s of the library's streaming-read probe over device buffers of the given sizes
    (each read `reps` times back to back); the ceiling is the best of them."""
    import torch
    import mla_latent_kv_absorbed_amd as M

    sink = torch.zeros(M.READ_PROBE_SINK_INTS, dtype=torch.int32, device="cuda")
    rates = {}
    for nbytes in sizes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        buf.fill_(7)
        for _ in range(2):
            M.mla_read_probe(buf, sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            M.mla_read_probe(buf, sink)
        b.record()
        torch.cuda.synchronize()
        rates[f"{nbytes >> 20}MiB"] = nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9
        del buf
        torch.cuda.empty_cache()
    return dict(kernel="read_probe", gbps_by_size=rates, gbps=max(rates.values()))


def run_prefill(L: int, Tq: int, steps: int, warmup: int, seed: int = 8):
    """Chunked prefill of one layer: Tq new tokens on an L-token context (the chunk's rows
    included), timed over `steps` calls; flops = expansion + attention of the visible tokens."""
    import torch
    from mla_latent_kv_absorbed_amd.workload import DevicePrefill

    dp = DevicePrefill(seed, L, Tq)
    li = dp.build_layer(0)
    out = torch.empty((Tq, 32, 128), dtype=torch.bfloat16, device=dp.dev)
    lse = torch.empty((Tq, 32), dtype=torch.float32, device=dp.dev)
    for _ in range(warmup):
        dp.run(li, out, lse)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dp.run(li, out, lse)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    visible = Tq * (L - Tq) + Tq * (Tq + 1) // 2
    flops_attn = visible * 32 * (192 + 128) * 2
    flops_expand = L * 512 * 8192 * 2
    tflops = (flops_attn + flops_expand) / (ms * 1e-3) / 1e12
    del li, dp, out, lse
    torch.cuda.empty_cache()
    return dict(workload=f"mla-prefill-chunk{Tq}-ctx{L}", context=L, chunk_tokens=Tq, ms_per_layer=ms,
                tokens_per_s=Tq / (ms * 1e-3), tflops_per_s=tflops, mfma_frac=tflops / MFMA_PEAK_TFLOPS,
                flops_per_call=flops_attn + flops_expand)


def library_reference(reps: int = 10):
    """Library rates on the prefill shapes, for context: torch.matmul (hipBLASLt) on the
    expansion GEMM [L x 512] x [512 x 8192] for L = 32768 and 131072, and torch's fused
    attention (flash and memory-efficient backends only; they need equal head dims, so V is
    padded to 192) on 4096 queries over 32768 keys without a mask."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    def timed(f, n):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    g = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    for L in (32768, 131072):
        c = torch.randn(L, 512, device="cuda", dtype=torch.bfloat16, generator=g)
        wt = torch.randn(512, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
        out = torch.empty(L, 8192, device="cuda", dtype=torch.bfloat16)
        ms = timed(lambda: torch.matmul(c, wt, out=out), reps)
        res[f"matmul_{L}x512x8192"] = dict(us=ms * 1e3, tflops_per_s=2 * L * 512 * 8192 / (ms * 1e-3) / 1e12)
        del c, wt, out
    q = torch.randn(1, 32, 4096, 192, device="cuda", dtype=torch.bfloat16, generator=g)
    k = torch.randn(1, 32, 32768, 192, device="cuda", dtype=torch.bfloat16, generator=g)
    v = torch.randn(1, 32, 32768, 192, device="cuda", dtype=torch.bfloat16, generator=g)
    for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([be]):
                ms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v), max(2, reps // 2))
            # useful flops: scores over 192 dims, values over the model's 128
            res[f"sdpa_{be.name.lower()}_q4096_k32768"] = dict(
                us=ms * 1e3, tflops_per_s=2 * 4096 * 32768 * 32 * (192 + 128) / (ms * 1e-3) / 1e12,
                note="V padded to 192; rate counts the 192 + 128 useful dims")
        except RuntimeError as e:
            res[f"sdpa_{be.name.lower()}_q4096_k32768"] = dict(unavailable=str(e)[:160])
    del q, k, v
    torch.cuda.empty_cache()
    return res


def cpu_baseline(k: int, budget_s: float = 15.0):
    """The un-absorbed fp64 oracle on the host cores, on a bounded sample of workload k.

    Sample: sequence 0, all 32 heads over its full context, layer after layer
    (each layer with its own inputs and kv_b_proj) until about budget_s of
    oracle time; the time per layer scales to one step (all layers, all
    sequences of the same length).  Input generation is not timed.
    """
    import numpy as np
    import threadpoolctl
    import oracle as O
    import synth
    from synth.configs import workload

    wl = workload(k)
    L, Sq, seed = wl.lens[0], wl.sq, wl.seed
    f = O.bf16_bits_to_float
    inv = O.yarn_inv_freq()
    scale = O.softmax_scale()
    layers, spent, spent_abs = 0, 0.0, 0.0
    while layers < wl.layers and spent < budget_s:
        c = f(synth.latent_bits(seed, layers, 0, 0, L))
        kk = O.round_to_bf16(O.rope_rotate(f(synth.kpe_bits(seed, layers, 0, 0, L)), np.arange(L), inv))
        qn = f(synth.qnope_bits(seed, layers, 0, Sq))
        qp = O.round_to_bf16(O.rope_rotate(f(synth.qpe_bits(seed, layers, 0, Sq)),
                                           (L - Sq + np.arange(Sq))[:, None], inv))
        w = f(synth.wkvb_bits(seed, layers))
        t0 = time.perf_counter()
        O.mla_attention_unabsorbed(qn, qp, c, kk, w, scale)
        spent += time.perf_counter() - t0
        t0 = time.perf_counter()
        O.mla_attention_absorbed(qn, qp, c, kk, w, scale)
        spent_abs += time.perf_counter() - t0
        layers += 1
    per_layer = spent / layers
    step_s = per_layer * wl.layers * wl.batch
    abs_step_s = spent_abs / layers * wl.layers * wl.batch
    threads = sum(p.get("num_threads", 0) for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas")
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count()
    return {"value": wl.batch * Sq / step_s, "unit": "tokens/s", "cores": host_cores, "blas_threads": threads,
            "kind": "oracle",
            "sample": (f"un-absorbed fp64 oracle, sequence 0 of {wl.name}, all 32 heads over the full {L}-token "
                       f"context, layers 0..{layers - 1}: {spent:.1f} s; {per_layer:.2f} s per layer scaled by "
                       f"{wl.layers} layers x {wl.batch} sequence(s) to one step"),
            "absorbed_reference": {"value": wl.batch * Sq / abs_step_s, "unit": "tokens/s",
                                   "s_per_layer": spent_abs / layers,
                                   "sample": "the absorbed fp64 CPU reference on the same layers and inputs"}}


def traffic_from_counters(workload_name: str):
    """HBM bytes per split-KV launch from committed rocprofv3 counters, if they were taken on
    this workload with this kernel source (else None)."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as fh:
        c = json.load(fh)
    if c.get("source_hash") != source_hash() or c.get("workload") != workload_name:
        return None
    return c.get("kernels", {}).get("splitkv_decode", {}).get("hbm_bytes_per_launch")


def _counter_rows(path):
    import csv
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = r.get("Kernel_Name", "")
            out.setdefault((r["Counter_Name"], name), []).append(float(r["Counter_Value"]))
    return out


def summarize_counters(fetch_csv: str, write_csv: str, copy_bytes: int, workload_name: str, command: str):
    """Writes profiles/splitkv_decode_counters.json from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch).  Each counter is scaled by what it reads for the calibration copy
    of copy_bytes bytes (the runtime's buffer-copy kernel) in the same run."""
    import statistics
    res = {"workload": workload_name, "source_hash": source_hash(), "command": command,
           "copy_bytes": copy_bytes, "kernels": {}}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        copy = [v for (cn, kn), vals in rows.items() if cn == counter and "copyBuffer" in kn for v in vals]
        copy_kib = max(copy) if copy else None      # the calibration copy is the largest buffer copy
        scale = (copy_bytes / 1024.0) / copy_kib if copy_kib else None
        res[f"{counter}_copy_kib"] = copy_kib
        res[f"{counter}_scale"] = scale
        for short, key in (("splitkv_decode", "splitkv_decode<"), ("combine_blocks", "combine_blocks"),
                           ("combine_one_row", "combine_one_row"), ("finalize_out", "finalize_out"),
                           ("prep_query", "prep_query")):
            vals = [v for (cn, kn), vs in rows.items() if cn == counter and key in kn for v in vs]
            if vals:
                kib = statistics.mean(vals)
                per.setdefault(short, {})[counter] = {"kib_per_dispatch": kib, "dispatches": len(vals),
                                                       "bytes_scaled": kib * 1024.0 * scale if scale else None}
    for short, d in per.items():
        f, w = d.get("FETCH_SIZE", {}), d.get("WRITE_SIZE", {})
        tot = None
        if f.get("bytes_scaled") is not None and w.get("bytes_scaled") is not None:
            tot = f["bytes_scaled"] + w["bytes_scaled"]
        res["kernels"][short] = {"fetch": f, "write": w, "hbm_bytes_per_launch": tot}
    with open(COUNTERS, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def counters_only(k: int, steps: int, layers: int, cache_dtype: str, kv_chunk):
    """A short run for hardware-counter passes: `layers` layers of workload k are built, then
    `steps` eager decode steps run over them (no graph, no timing).  The build needs few
    dispatches (the slot tensors are made once per chunk with no dtype casts), and a counter
    pass restricted to the decode kernels by name collects nothing while it runs."""
    import torch
    from mla_latent_kv_absorbed_amd.workload import DeviceWorkload
    from synth.configs import workload

    wl = workload(k)
    dw = DeviceWorkload(wl, kv_chunk=kv_chunk, cache_dtype=cache_dtype)
    lis = [dw.build_layer(l) for l in range(layers)]
    torch.cuda.synchronize()
    log(f"[counters] built {layers} layer(s) of {wl.name} ({cache_dtype}, chunk {dw.chunk_used})")
    out = torch.empty((dw.B, dw.Sq, 32, 128), dtype=torch.bfloat16, device=dw.dev)
    lse = torch.empty((dw.B, dw.Sq, 32), dtype=torch.float32, device=dw.dev)
    for s in range(steps):
        for li in lis:
            dw.step(li, out=out, lse=lse)
        torch.cuda.synchronize()
        log(f"[counters] step {s + 1}/{steps} done")
    print(json.dumps({"counters_run": wl.name, "cache_dtype": cache_dtype, "layers": layers, "steps": steps,
                      "kv_chunk": dw.chunk_used, "tokens": sum(dw.lens), "query_tokens": dw.Sq,
                      "visible_token_queries": sum(L * dw.Sq - dw.Sq * (dw.Sq - 1) // 2 for L in dw.lens)}),
          flush=True)


def _short_kernel(name: str) -> str:
    n = name.replace("void ", "").replace("mla::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0]


def summarize_pmc(paths, title: str, command: str):
    """Markdown table of rocprofv3 --pmc CSVs of one workload (several passes may be given): per
    kernel, the mean of each counter per dispatch, and where the counters are present the MFMA
    busy share SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs), GRBM_GUI_ACTIVE being
    summed over the XCDs and the busy cycles over the SIMDs."""
    import csv
    import statistics
    rows, dur = {}, {}
    simds, xccs = None, None
    for path in paths:
        for (cn, kn), vals in _counter_rows(path).items():
            rows.setdefault(_short_kernel(kn), {}).setdefault(cn, []).extend(vals)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                dur.setdefault(_short_kernel(r["Kernel_Name"]), []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        info = os.path.join(os.path.dirname(path), "run_agent_info.csv")
        if os.path.exists(info):
            with open(info) as fh:
                for r in csv.DictReader(fh):
                    if r.get("Name", "").startswith("gfx"):
                        simds, xccs = int(r["Simd_Count"]), int(r["Num_Xcc"])
    lines = [f"# {title}", "", "Commands (repository root, one MI355X; one counter pass per run):", ""]
    lines += ["    " + c for c in command.split(" ;; ")]
    lines += ["", f"Device: {simds} SIMDs, {xccs} XCDs (run_agent_info.csv).", ""]
    counters = sorted({cn for d in rows.values() for cn in d})
    lines.append("| kernel | dispatches | median us | " + " | ".join(counters) + " | MFMA busy |")
    lines.append("|---|---:|---:|" + "---:|" * len(counters) + "---:|")
    for kn in sorted(rows):
        d = rows[kn]
        n = max(len(v) for v in d.values())
        cells = [f"{statistics.mean(d[c]):,.0f}" if c in d else "" for c in counters]
        busy = ""
        if simds and xccs and "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d:
            cyc = statistics.mean(d["GRBM_GUI_ACTIVE"]) / xccs
            busy = f"{statistics.mean(d['SQ_VALU_MFMA_BUSY_CYCLES']) / (simds * cyc):.1%}"
        lines.append(f"| {kn} | {n // max(1, len(paths))} | {statistics.median(dur[kn]):.1f} | " + " | ".join(cells)
                     + f" | {busy} |")
    print("\n".join(lines))


def summarize_trace(path: str, title: str, command: str, splitkv: str):
    """Markdown summary of a rocprofv3 --kernel-trace CSV: per kernel the calls and durations, and
    the median durations over back-to-back layer sequences (prep_query -> the split-KV kernel whose
    name starts with `splitkv` -> the combine (combine_one_row or combine_blocks<RB>) -> finalize_out,
    gaps under 2 us)."""
    import csv
    import statistics
    ks = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            ks.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short_kernel(r["Kernel_Name"])))
    ks.sort()
    per = {}
    for a, b, n in ks:
        per.setdefault(n, []).append((b - a) / 1e3)
    total = sum(sum(v) for v in per.values())
    lines = [f"# {title}", "", "Command (repository root, one MI355X):", "", "    " + command, "",
             "| kernel | calls | avg us | median us | min us | max us | share |", "|---|---:|---:|---:|---:|---:|---:|"]
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {n[:70]} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} | "
                     f"{max(v):.2f} | {sum(v) / total:.1%} |")
    seq = {"prep_query": [], "split": [], "combine": [], "finalize_out": [], "layer": []}
    combine_names = set()
    for i in range(len(ks) - 3):
        names = [ks[i + k][2] for k in range(4)]
        if names[0] != "prep_query" or not names[1].startswith(splitkv) or not names[2].startswith("combine") \
                or names[3] != "finalize_out":
            continue
        if any(ks[i + k + 1][0] - ks[i + k][1] > 2000 for k in range(3)):
            continue
        combine_names.add(names[2])
        for k, key in enumerate(("prep_query", "split", "combine", "finalize_out")):
            seq[key].append((ks[i + k][1] - ks[i + k][0]) / 1e3)
        seq["layer"].append((ks[i + 3][1] - ks[i][0]) / 1e3)
    if seq["layer"]:
        comb = " / ".join(sorted(combine_names))
        lines += ["", f"Back-to-back layer sequences (prep_query -> {splitkv}* -> {comb} -> finalize_out, "
                      f"gaps < 2 us; {len(seq['layer'])} found), median durations:", "", "| kernel | median us |",
                  "|---|---:|"]
        for key in ("prep_query", "split", "combine", "finalize_out"):
            label = {"split": splitkv, "combine": comb}.get(key, key)
            lines.append(f"| {label} | {statistics.median(seq[key]):.2f} |")
        lines.append(f"| one layer, first start to last end | {statistics.median(seq['layer']):.2f} |")
    print("\n".join(lines))


def copy_calibration(nbytes: int):
    """A plain device-to-device copy of nbytes, three times (a known-size reference for counters)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index (1 = 32K, 3 = 256K)")
    ap.add_argument("--kv-chunk", type=int, default=None,
                    help="tokens per split for the main workload (0: device-balanced; default: the workload's own)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-256k", action="store_true", help="skip the 256K report")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit cache report")
    ap.add_argument("--no-more", action="store_true",
                    help="skip the report on the other workloads (batched paged, speculative verify, 512K)")
    ap.add_argument("--library-reference", action="store_true",
                    help="run only the library rates on the prefill shapes (hipBLASLt GEMM, torch fused attention) and print them")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the chunked-prefill report (4096 new tokens on 32K and 128K contexts) and print it")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="first copy this many MiB device-to-device 3 times (reference for rocprofv3 counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/splitkv_decode_counters.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--counters-command", default="", help="command line recorded with --summarize-counters")
    ap.add_argument("--counters-only", action="store_true",
                    help="build --counter-layers layers of --config and run --steps eager decode steps, nothing else "
                         "(for hardware-counter passes)")
    ap.add_argument("--counter-layers", type=int, default=1)
    ap.add_argument("--cache-dtype", default="bf16", choices=("bf16", "fp8"),
                    help="cache format of the main workload (and of --counters-only)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print a markdown table (mean per dispatch, per kernel and counter) of rocprofv3 --pmc CSVs")
    ap.add_argument("--pmc-title", default="rocprofv3 counters")
    ap.add_argument("--summarize-trace", metavar="CSV", help="print a markdown summary of a rocprofv3 kernel trace")
    ap.add_argument("--trace-splitkv", default="splitkv_decode<", help="split-KV kernel name prefix for the layer table")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.pmc_title, args.counters_command)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.pmc_title, args.counters_command, args.trace_splitkv)
        return
    if args.summarize_counters:
        from synth.configs import workload
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1],
                           args.copy_calibration_mb << 20, workload(args.config).name, args.counters_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()
    if args.counters_only:
        counters_only(args.config, args.steps, args.counter_layers, args.cache_dtype, args.kv_chunk)
        return
    if args.library_reference:
        print(json.dumps({"library_reference": library_reference()}), flush=True)
        return
    if args.prefill_only:
        res = {}
        for L, Tq in ((32768, 4096), (131072, 4096)):
            r = run_prefill(L, Tq, args.steps, args.warmup)
            res[r["workload"]] = r
        print(json.dumps({"prefill": res}), flush=True)
        return
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb << 20)
    main_res = run_workload(args.config, args.steps, args.warmup, not args.no_graph, kv_chunk=args.kv_chunk,
                            label=f"config{args.config}", cache_dtype=args.cache_dtype)
    log(f"[config{args.config}] {json.dumps(main_res)}")
    extra = None
    if not args.no_256k and args.config != 3:
        extra = {}
        for name, chunk in (("kv_chunk_4096", 4096), ("kv_chunk_auto", 0)):
            r = run_workload(3, max(3, min(args.steps, 10)), 2, not args.no_graph, kv_chunk=chunk, label=f"256k-{name}")
            log(f"[256k {name}] {json.dumps(r)}")
            extra[name] = {k: r[k] for k in ("tokens_per_s", "ms_per_step", "step_latent_gbps", "kernel_avg_us",
                                            "kernel_latent_gbps", "kernel_tflops", "kv_chunk")}
            extra[name]["kernel_hbm_frac"] = r["kernel_latent_gbps"] / HBM_PEAK_GBPS
    fp8 = None
    if not args.no_fp8:
        fp8 = {}
        for name, k in (("ctx32k", 1), ("ctx256k", 3)):
            if args.no_256k and k == 3:
                continue
            r = run_workload(k, max(3, min(args.steps, 10)), 2, not args.no_graph, kv_chunk=0, label=f"fp8-{name}",
                             cache_dtype="fp8")
            log(f"[fp8 {name}] {json.dumps(r)}")
            fp8[name] = {key: r[key] for key in ("workload", "tokens_per_s", "ms_per_step", "step_latent_gbps",
                                               "kernel_avg_us", "kernel_latent_gbps", "kernel_tflops", "kv_chunk")}
            fp8[name]["kernel_hbm_frac"] = r["kernel_latent_gbps"] / HBM_PEAK_GBPS
    more = None
    if not args.no_more:
        more = {}
        for k in (2, 4, 7, 5, 6):
            if k == args.config:
                continue
            r = run_workload(k, max(3, min(args.steps, 10)), 2, not args.no_graph, kv_chunk=0, label=f"config{k}")
            log(f"[config{k}] {json.dumps(r)}")
            more[r["workload"]] = {key: r[key] for key in ("batch", "query_tokens", "layout", "tokens_per_s",
                                                         "ms_per_step", "step_latent_gbps", "kernel_avg_us",
                                                         "kernel_latent_gbps", "kernel_tflops", "kv_chunk")}
            more[r["workload"]]["kernel_hbm_frac"] = r["kernel_latent_gbps"] / HBM_PEAK_GBPS
            more[r["workload"]]["kernel_mfma_frac"] = r["kernel_tflops"] / MFMA_PEAK_TFLOPS
        if not args.no_fp8:
            # speculative verify over the 8-bit cache (656 B per token and layer)
            r = run_workload(4, max(3, min(args.steps, 10)), 2, not args.no_graph, kv_chunk=0, label="fp8-config4",
                             cache_dtype="fp8")
            log(f"[fp8 config4] {json.dumps(r)}")
            key = r["workload"] + "-fp8"
            more[key] = {k: r[k] for k in ("batch", "query_tokens", "layout", "tokens_per_s", "ms_per_step",
                                           "step_latent_gbps", "kernel_avg_us", "kernel_latent_gbps",
                                           "kernel_tflops", "kv_chunk")}
            more[key]["cache_dtype"] = "fp8"
            more[key]["kernel_hbm_frac"] = r["kernel_latent_gbps"] / HBM_PEAK_GBPS
            more[key]["kernel_mfma_frac"] = r["kernel_tflops"] / MFMA_PEAK_TFLOPS
    prefill = None
    if not args.no_more:
        prefill = {}
        for L, Tq in ((32768, 4096), (131072, 4096)):
            r = run_prefill(L, Tq, 5, 2)
            log(f"[prefill {Tq}/{L}] {json.dumps(r)}")
            prefill[r["workload"]] = r
    latency = None
    if not args.no_more:
        latency = {}
        for name, chunk in (("kv_chunk_auto", 0), ("one_split", 1024)):
            r = run_latency(0, chunk)
            log(f"[config0 {name}] {json.dumps(r)}")
            latency[name] = r
    ceiling = None
    if not args.no_more:
        ceiling = read_ceiling()
        ceiling["splitkv_frac_of_ceiling"] = main_res["kernel_latent_gbps"] / ceiling["gbps"]
        log(f"[read ceiling] {json.dumps(ceiling)}")
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.config)

    bpl = main_res["kernel_bytes_per_launch"]
    achieved = main_res["kernel_latent_gbps"]
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) latents, rope keys and queries, N(0,1/512) kv_b_proj per layer; no trained weights",
        "config": {k: main_res[k] for k in ("workload", "batch", "query_tokens", "context", "layers", "layout",
                                           "kv_chunk", "graph")},
        "latent_gbps_step": main_res["step_latent_gbps"],
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_from_counters(main_res["workload"]),
            "kernel": "splitkv_decode", "bytes_per_launch": bpl, "avg_launch_us": main_res["kernel_avg_us"],
        },
        "cpu_baseline": cpu,
        "kernel_tflops": main_res["kernel_tflops"],
        "read_ceiling": ceiling,
        "ctx1k_one_layer": latency,
        "ctx256k": extra,
        "fp8_cache": fp8,
        "other_workloads": more,
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
