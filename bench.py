#!/usr/bin/env python3
"""Benchmark of NVFP4 paged decode attention on one MI355X.

One step = one decode step of one layer for the whole batch, every decode row of
the hot path: quantize-on-write of the step's new K/V token of every sequence
into the NVFP4 pool, the split-K decode kernel that reads the batch's whole NVFP4
cache and dequantizes it in registers, and the split combine. The step is the
fused call (the split launch writes the new tokens before reading their pages,
then the combine); the same step as three launches (quantize, split, combine) is
timed beside it as step_three_launch_ms, the two alternating. Inputs (pool, Q,
page table, the new tokens) are resident in HBM before the timed region; the
pool is filled once beforehand by the same quantize kernel from seeded
synthetic K/V. The new token of sequence b is its last token (index L_b - 1),
so each step rewrites the same bytes and every step attends over L_b tokens.

The headline workload is the largest single-GPU decode configuration, batch 15
x 163840 tokens (2.83 GB of NVFP4 K/V read per step). The same JSON line carries
every other workload (``workloads``: the tiny case, batch 44 x 32K, the ragged
batch 70, and batch 2 x 1M with its chunked-prefill extend step), the FP8 E4M3
cache on each (matched batch), and the capacity comparison (``capacity``): FP8
at the resident counts the pages report for it (44, 10, 1 at 32K, 160K, 1M)
against NVFP4 at its own (70, 15, 2).

Prints one JSON line:
  value         KV-read GB/s = algorithmic NVFP4 K+V bytes read per step / time per step
  roofline      the decode split kernel (the dominant kernel) against MI355X HBM peak:
                algorithmic bytes per launch / its average duration, both from HIP
                events recorded on its stream inside the timed region
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16/fp16 matrix peak
METRIC = "NVFP4 paged decode-attn KV-read GB/s (% of HBM peak) + decode steps/s/layer"
HEADLINE = 4  # batch 15 x 163840: the largest decode workload that fits one GPU
# Resident requests the pages report at 32K, 160K and 1M tokens: FP8 -> NVFP4.
CAPACITY = ((32768, 44, 70), (163840, 10, 15), (1048576, 1, 2))
# The pages' peak-batch decode gains once NVFP4 holds more requests (context only:
# end-to-end serving on one RTX PRO 6000 Blackwell, not a kernel measure).
CAPACITY_PAGES_GAIN = {32768: "+37.37%", 163840: "+57.75%", 1048576: "+78.46%"}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE,
                    help="headline workload 1..5 (default 4: batch 15 x 163840, the largest decode workload)")
    ap.add_argument("--workloads", default="1,2,3,5",
                    help="other workloads measured in the same run (comma list; empty for none)")
    ap.add_argument("--splits", type=int, default=-1, help="-1 = the workload's setting, else the library default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8-baseline", action="store_true",
                    help="skip the FP8 E4M3 cache timed on the same workloads and step")
    ap.add_argument("--no-capacity", action="store_true", help="skip the capacity-driven FP8 comparison")
    ap.add_argument("--cpu-sample-tokens", type=int, default=786432,
                    help="tokens of the headline workload the CPU oracle attends over (whole sequences, >= 1)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration only: time a plain device copy of this many bytes instead of the decode step "
                         "(the reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--trace-summary", default="",
                    help="no GPU work: summarize a rocprofv3 --kernel-trace output directory of a bench.py run "
                         "(per kernel: every launch, and the launches after the first --trace-skip of each)")
    ap.add_argument("--trace-skip", type=int, default=0)
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="with --trace-summary: the traced run's --steps, to group its decode launches by phase")
    ap.add_argument("--trace-warmup", type=int, default=0, help="with --trace-steps: the traced run's --warmup")
    return ap.parse_args(argv)


def copy_calibration(nbytes, steps):
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes": src.numel() * 4, "ms": round(ms, 4),
                      "GBps_read_plus_write": round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)


def decode_phases(launches, steps, warmup):
    """The headline decode step's launches grouped the way decode_step() issues
    them: ``warmup`` pairs of one fused and one three-launch step, three passes
    of ``steps`` fused then ``steps`` three-launch steps, then the
    kernel-timing pass of ``steps`` fused steps. ``launches`` is (kernel, start
    ns, end ns) in start order; a fused step is split + combine, a three-launch
    step is quantize + split + combine. Per phase: mean, min and max of the
    split kernel, the mean combine and new-token quantize, and the mean span of
    a step from its first kernel's start to its last kernel's end (in us).
    Returns [] when the trace does not hold the whole sequence."""
    import statistics

    first = next((i for i, x in enumerate(launches) if x[0] == "k_decode_split"), None)
    if first is None:
        return []
    seq = [x for x in launches[first:] if x[0] in ("k_decode_split", "k_decode_combine", "k_quantize")]
    grouped, i = [], 0
    while i < len(seq):
        names = tuple(x[0] for x in seq[i:i + 3])
        if names == ("k_quantize", "k_decode_split", "k_decode_combine"):
            grouped.append(seq[i:i + 3])
            i += 3
        elif names[:2] == ("k_decode_split", "k_decode_combine"):
            grouped.append(seq[i:i + 2])
            i += 2
        else:
            break  # the decode steps end at the first launch that is not part of one
    plan = [("warm-up, fused and three-launch in turn", 2 * warmup)]
    for p in range(3):
        plan += [(f"pass {p}, fused", steps), (f"pass {p}, three-launch", steps)]
    plan.append(("kernel-timing pass (fused)", steps))
    if len(grouped) < sum(n for _, n in plan):
        return []
    out, k = [], 0

    def us(v):
        return round(statistics.mean(v) / 1000, 1) if v else None

    for label, n in plan:
        grp = grouped[k:k + n]
        k += n
        dur = {name: [e - s for g in grp for (nm, s, e) in g if nm == name]
               for name in ("k_decode_split", "k_decode_combine", "k_quantize")}
        sp = dur["k_decode_split"]
        out.append({"phase": label, "steps": n, "split_mean_us": us(sp), "split_min_us": round(min(sp) / 1000, 1),
                    "split_max_us": round(max(sp) / 1000, 1), "combine_mean_us": us(dur["k_decode_combine"]),
                    "quantize_mean_us": us(dur["k_quantize"]),
                    "step_span_mean_us": us([g[-1][2] - g[0][1] for g in grp])})
    return out


def trace_summary(path, skip, steps=0, warmup=0):
    """Per-kernel durations from a rocprofv3 kernel-trace CSV under ``path``:
    all launches, and the launches after the first ``skip`` of each kernel
    (launches keep their dispatch order), with the grid they ran on. With
    ``steps`` > 0, also the headline decode step's launches by phase (the
    bench.py run's --steps and --warmup)."""
    import csv
    import glob
    import statistics

    files = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {path}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per, launches = {}, []
    for r in rows:
        m = re.search(r"\b(k_[A-Za-z0-9_]+)\s*[(<]", r["Kernel_Name"])  # the library's kernels are k_*
        if not m:
            continue
        name = m.group(1)
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        launches.append((name, t0, t1))
        per.setdefault(name, []).append((t1 - t0, r.get("Grid_Size_X", r.get("Grid_Size", ""))))
    out = {}
    for name, v in per.items():
        d = [x for x, _ in v]
        steady = d[skip:] if len(d) > skip else d
        out[name] = {"launches": len(d), "mean_ns": round(statistics.mean(d)), "min_ns": min(d), "max_ns": max(d),
                     "steady_launches": len(steady), "steady_mean_ns": round(statistics.mean(steady)),
                     "steady_median_ns": round(statistics.median(steady)), "grids": sorted({g for _, g in v})}
    if steps > 0:
        out["decode_phases"] = decode_phases(launches, steps, warmup)
    print(json.dumps(out, indent=1))


def committed_traffic(workload, splits, kernel="k_decode_split"):
    """HBM bytes per split-kernel launch from the committed rocprofv3 counter
    summary in profiles/, or None when there is none for this kernel, workload
    and split count or when the kernel source has changed since the counters
    were taken."""
    import glob
    import hashlib

    here = os.path.dirname(os.path.abspath(__file__))
    for path in glob.glob(os.path.join(here, "profiles", "k_decode_split*_traffic.md")):
        fields = {}
        for line in open(path):
            if ":" in line and line.startswith("    "):
                k, v = line.strip().split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("kernel") != kernel:
            continue
        if fields.get("workload") != workload or fields.get("num_splits") != str(splits):
            continue
        # every source file the kernel is compiled from, hashed in the listed order
        srcs = [os.path.join(here, f.strip()) for f in fields.get("kernel_source", "").split(",") if f.strip()]
        if not srcs or not all(os.path.isfile(f) for f in srcs):
            continue
        h = hashlib.sha256()
        for f in srcs:
            h.update(open(f, "rb").read())
        if h.hexdigest() == fields.get("kernel_source_sha256"):
            return int(fields["traffic_bytes_per_launch"])
        # taken on other kernel sources: look on
    return None


def fill_pool(w, pool, B, W, torch, seqs=None, step=65536, fp8=False):
    """Quantize-on-write every listed sequence's K/V into the pool (library kernel)."""
    quant = B.fp8_kv_quantize if fp8 else B.nvfp4_kv_quantize
    for b in (range(w.batch) if seqs is None else seqs):
        L = int(w.seq_lens[b])
        for t0 in range(0, L, step):
            t1 = min(L, t0 + step)
            k, v = W.kv(w, b, t0, t1, device="cuda")
            quant(k, v, torch.as_tensor(W.slots(w, b, t0, t1), device="cuda"), pool)
    torch.cuda.synchronize()


def step_inputs(w, W, torch):
    """Q, page table, lengths and the step's new token of every sequence (its
    last one) on the device."""
    q = W.query(w, device="cuda")
    pt = torch.as_tensor(w.page_table[:w.batch], device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    new_k, new_v, new_slots = [], [], []
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        k, v = W.kv(w, b, L - 1, L, device="cuda")
        new_k.append(k)
        new_v.append(v)
        new_slots.append(int(W.slots(w, b, L - 1, L)[0]))
    new_k = torch.cat(new_k).contiguous()
    new_v = torch.cat(new_v).contiguous()
    new_slots = torch.tensor(new_slots, dtype=torch.int32, device="cuda")
    return q, pt, sl, new_k, new_v, new_slots


def timed_loop(torch, stream, fn, n):
    """n calls back to back, events only around the whole loop (an event recorded
    between two kernels holds the second one back by several us). Returns ms per
    call and the host wall time of the region."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(n):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n, time.perf_counter() - t0


def decode_step(w, pool, splits, B, W, torch, steps, warmup, fp8=False, three_launch=True):
    """Times the fused decode step (and, unless fp8, the three-launch form beside
    it, the two alternating over three passes of ``steps`` steps; medians), then
    the split kernel alone: ``steps`` more fused steps, each split launch
    bracketed by events on the stream it runs on."""
    q, pt, sl, new_k, new_v, new_slots = step_inputs(w, W, torch)
    ws = torch.empty(B.nvfp4_paged_decode_attn_workspace_bytes(w.batch, w.num_q_heads, splits), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    append = B.fp8_paged_decode_attn_append if fp8 else B.nvfp4_paged_decode_attn_append

    def step(_=0, evs=None):
        if not evs:
            append(q, new_k, new_v, pt, sl, pool, w.sm_scale, w.max_seq_len, splits, ws, out=out, stream=stream)
            return
        evs[0].record(stream)
        append(q, new_k, new_v, pt, sl, pool, w.sm_scale, w.max_seq_len, splits, ws, stream=stream, combine=False)
        evs[1].record(stream)
        B.nvfp4_decode_combine(ws, w.batch, w.num_q_heads, splits, out, stream=stream)

    def step_three(_=0):
        # the same step as three launches: quantize-on-write, split kernel, combine
        B.nvfp4_kv_quantize(new_k, new_v, new_slots, pool, stream=stream)
        B.nvfp4_paged_decode_attn_partial(q, pt, sl, pool, w.sm_scale, w.max_seq_len, splits, ws, stream=stream)
        B.nvfp4_decode_combine(ws, w.batch, w.num_q_heads, splits, out, stream=stream)

    three = three_launch and not fp8
    for _ in range(warmup):
        step()
        if three:
            step_three()
    runs, runs_three = [], []
    for _ in range(3):
        runs.append(timed_loop(torch, stream, step, steps))
        if three:
            runs_three.append(timed_loop(torch, stream, step_three, steps)[0])
    runs.sort()
    ms, wall = runs[1]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        step(evs=kev[i])
    torch.cuda.synchronize()
    k_ms = sum(a.elapsed_time(b) for a, b in kev) / steps
    r = {"ms": ms, "k_ms": k_ms, "wall": wall}
    if three:
        r["ms_three"] = sorted(runs_three)[1]
    return r


def fp8_row(w, splits, B, W, torch, steps, warmup, nvfp4_ms=None, nvfp4_k_ms=None):
    """The same decode step over an FP8 E4M3 cache of the same K/V (the format the
    pages compare NVFP4 against), through the same fused call."""
    pool8 = B.Fp8Pool(w.num_pages, w.num_kv_heads, device="cuda")
    fill_pool(w, pool8, B, W, torch, fp8=True)
    t = decode_step(w, pool8, splits, B, W, torch, steps, warmup, fp8=True)
    del pool8
    torch.cuda.empty_cache()
    kv8 = int(w.seq_lens.astype("int64").sum()) * w.num_kv_heads * 2 * 128  # one byte per value
    r = {"kv_bytes_per_step": kv8, "ms_per_step": round(t["ms"], 5), "GBps": round(kv8 / (t["ms"] * 1e-3) / 1e9, 2),
         "kernel": "k_decode_split_fp8", "kernel_ms": round(t["k_ms"], 5),
         "kernel_GBps": round(kv8 / (t["k_ms"] * 1e-3) / 1e9, 2),
         "kernel_frac": round(kv8 / (t["k_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "num_splits": splits,
         "tokens_per_s_per_layer": round(w.batch * 1e3 / t["ms"], 1),
         "nvfp4_bytes_over_fp8": round(w.kv_bytes_per_step() / kv8, 4)}
    if nvfp4_ms:
        r["nvfp4_step_speedup"] = round(t["ms"] / nvfp4_ms, 3)
        r["nvfp4_kernel_speedup"] = round(t["k_ms"] / nvfp4_k_ms, 3)
    return r


def cpu_baseline(w, sample_tokens, W, torch):
    """The oracle (fp64 attention over its own NVFP4 quantization of the same
    seeded K/V) on the first whole sequences that fit ``sample_tokens`` (at least
    one), all heads. Only the decode attention is timed; the sample's KV bytes
    over that time give a GB/s figure."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    n_seqs, tok = 0, 0
    while n_seqs < w.batch and (n_seqs == 0 or tok + int(w.seq_lens[n_seqs]) <= sample_tokens):
        tok += int(w.seq_lens[n_seqs])
        n_seqs += 1
    lens = w.seq_lens[:n_seqs]
    sub = W.Workload(name=w.name, seed=w.seed, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                     seq_lens=lens, page_table=w.page_table[:n_seqs], num_pages=w.num_pages,
                     outlier_channels=w.outlier_channels)
    pool = np.zeros(oracle.pool_bytes(w.num_pages, w.num_kv_heads), dtype=np.uint8)
    for b in range(n_seqs):
        L = int(lens[b])
        for t0 in range(0, L, 65536):
            t1 = min(L, t0 + 65536)
            k, v = W.kv(w, b, t0, t1, device="cuda")
            oracle.quantize_to_pool(k.cpu().numpy(), v.cpu().numpy(), W.slots(w, b, t0, t1), w.num_pages,
                                    pool=pool, n_threads=cores)
            del k, v
    q = W.query(w, device="cuda")[:n_seqs].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    oracle.decode_attn(q, sub.page_table, lens, pool, w.num_kv_heads, w.sm_scale, n_threads=cores)
    dt = time.perf_counter() - t0
    kv_bytes = sub.kv_bytes_per_step()
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_seqs} of {w.batch} sequences, all {w.num_q_heads} query heads ({int(lens.sum())} tokens, "
                      f"{kv_bytes} KV bytes): fp64 decode attention over the oracle's own NVFP4 cache, {dt:.2f} s",
            "seconds": round(dt, 3),
            "decode_steps_per_s_per_layer_equiv": round((kv_bytes / w.kv_bytes_per_step()) / dt, 6)}


def cpu_extend_baseline(w, W, torch, prefix_sample=16384):
    """The oracle on the extend path of the chunked-prefill workload: quantize of
    the whole 8192-token bf16 chunk, and dequantization (fp64) of the first
    prefix_sample tokens of the cached prefix, with all host cores. Bytes are the
    GPU kernels' algorithmic bytes for the same tokens."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    row, P, C, H = w.extend_row, w.extend_prefix, w.extend_chunk, w.num_kv_heads
    kc, vc = W.extend_chunk_kv(w)
    kb = kc.contiguous().view(torch.int16).numpy().view(np.uint16)
    vb = vc.contiguous().view(torch.int16).numpy().view(np.uint16)
    pool = np.zeros(oracle.pool_bytes(w.num_pages, H), dtype=np.uint8)
    reps = 10  # one pass takes tens of ms on many cores
    cslots = W.slots(w, row, P, P + C)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.quantize_to_pool(kb, vb, cslots, w.num_pages, pool=pool, n_threads=cores)
    dq = (time.perf_counter() - t0) / reps
    q_bytes = C * H * 128 * 2 * 2 + C * H * 2 * 8 * 9
    n = min(prefix_sample, P)
    k, v = W.kv(w, row, 0, n)
    oracle.quantize_to_pool(k.numpy(), v.numpy(), W.slots(w, row, 0, n), w.num_pages, pool=pool, n_threads=cores)
    pt = np.ascontiguousarray(w.page_table[row:row + 1, :-(-n // 16)])
    t0 = time.perf_counter()
    oracle.dequant_workspace(pool, H, pt, np.array([n], dtype=np.int32))
    dd = time.perf_counter() - t0
    d_bytes = n * H * 2 * 8 * 9 + n * H * 128 * 2 * 2
    return {"quantize_chunk": {"value": round(q_bytes / dq / 1e9, 4), "unit": "GB/s", "seconds": round(dq, 3),
                               "sample": f"the whole {C}-token bf16 chunk, {H} KV heads (mean of {reps} passes)"},
            "dequant_prefix": {"value": round(d_bytes / dd / 1e9, 4), "unit": "GB/s", "seconds": round(dd, 3),
                               "sample": f"the first {n} of {P} prefix tokens, {H} KV heads, fp64 output "
                                         "(bytes counted as the GPU's bf16 workspace)"},
            "cores": cores, "kind": "oracle"}


def extend_step(w, pool, B, W, torch, steps, warmup):
    """The chunked-prefill step of the 1M workload: quantize-write the 8192-token
    bf16 chunk into the extend request's pages, dequantize its 163840-token prefix
    into a bf16 (and, separately, an FP8) workspace, and run the chunk's attention
    over workspace + chunk. Each kernel is timed over its own back-to-back
    launches; the step times are sums of those averages."""
    row = w.extend_row
    # the prefix must be resident: fill it once (untimed)
    P, C = w.extend_prefix, w.extend_chunk
    fill_pool_rows(w, pool, B, W, torch, row, P)
    kc, vc = W.extend_chunk_kv(w, device="cuda")
    qc = W.extend_query(w, device="cuda")
    att_out = torch.empty_like(qc)
    cslots = torch.as_tensor(W.slots(w, row, P, P + C), device="cuda")
    # Two prefixes of P tokens in turn, the extend request's and the first P tokens
    # of decode sequence 0 (both in the pool), so that one repeat's 189 MB read is
    # not served from the 256 MB last-level cache left by the previous one.
    n_pp = -(-P // 16)
    pts = [torch.as_tensor(w.page_table[r:r + 1, :n_pp], device="cuda").contiguous() for r in (row, 0)]
    sl = torch.tensor([P], dtype=torch.int32, device="cuda")
    ro = torch.zeros(1, dtype=torch.int64, device="cuda")
    k_ws = torch.empty((P, w.num_kv_heads, 128), dtype=torch.bfloat16, device="cuda")
    v_ws = torch.empty_like(k_ws)
    k_w8 = torch.empty((P, w.num_kv_heads, 128), dtype=torch.float8_e4m3fn, device="cuda")
    v_w8 = torch.empty_like(k_w8)
    k_wt = torch.empty_like(k_ws)  # the tiled workspace: bf16 K rows, f16 V^T tiles
    v_wt = B.tiled_v_workspace(P, w.num_kv_heads)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    for i in range(warmup):
        B.nvfp4_kv_quantize(kc, vc, cslots, pool, stream=stream)
        B.nvfp4_kv_dequant_workspace(pool, pts[i % 2], sl, ro, P, k_ws, v_ws, stream=stream)
        B.nvfp4_extend_attn(qc, k_ws, v_ws, kc, vc, w.sm_scale, out=att_out, stream=stream)

    def loop(fn, n):
        return timed_loop(torch, stream, fn, n)[0]

    n_small = max(10, 4 * steps)
    n_att = max(2, steps)
    # quantize-write of the chunk (rewrites the same pages each time)
    q_ms = loop(lambda i: B.nvfp4_kv_quantize(kc, vc, cslots, pool, stream=stream), n_small)
    # prefix dequant, the two prefixes in turn
    d_ms = loop(lambda i: B.nvfp4_kv_dequant_workspace(pool, pts[i % 2], sl, ro, P, k_ws, v_ws, stream=stream), n_small)
    d8_ms = loop(lambda i: B.nvfp4_kv_dequant_workspace(pool, pts[i % 2], sl, ro, P, k_w8, v_w8, stream=stream),
                 n_small)
    dt_ms = loop(lambda i: B.nvfp4_kv_dequant_workspace(pool, pts[i % 2], sl, ro, P, k_wt, v_wt, stream=stream),
                 n_small)
    # attention over the bf16 and the FP8 workspace, then the fused prefill path
    # (attention that also quantize-writes the chunk)
    B.nvfp4_kv_dequant_workspace(pool, pts[0], sl, ro, P, k_ws, v_ws, stream=stream)
    B.nvfp4_kv_dequant_workspace(pool, pts[0], sl, ro, P, k_w8, v_w8, stream=stream)
    B.nvfp4_kv_dequant_workspace(pool, pts[0], sl, ro, P, k_wt, v_wt, stream=stream)
    at_ms = loop(lambda i: B.nvfp4_extend_attn(qc, k_wt, v_wt, kc, vc, w.sm_scale, out=att_out, stream=stream), n_att)
    a_ms = loop(lambda i: B.nvfp4_extend_attn(qc, k_ws, v_ws, kc, vc, w.sm_scale, out=att_out, stream=stream), n_att)
    a8_ms = loop(lambda i: B.nvfp4_extend_attn(qc, k_w8, v_w8, kc, vc, w.sm_scale, out=att_out, stream=stream), n_att)
    af_ms = loop(lambda i: B.nvfp4_extend_attn(qc, k_ws, v_ws, kc, vc, w.sm_scale, out=att_out, chunk_pool=pool,
                                               chunk_slots=cslots, stream=stream), n_att)
    del k_ws, v_ws, k_w8, v_w8, k_wt, v_wt
    # attention flops: QK^T and PV, 2 x 128 multiply-adds per (query row, visible key)
    a_flops = 4 * w.num_q_heads * 128 * (C * P + C * (C + 1) // 2)
    q_bytes = C * w.num_kv_heads * 128 * 2 * 2 + C * w.num_kv_heads * 2 * 8 * 9  # bf16 in + NVFP4 out
    d_bytes = P * w.num_kv_heads * 2 * 8 * 9 + P * w.num_kv_heads * 128 * 2 * 2  # NVFP4 in + bf16 out
    d8_bytes = P * w.num_kv_heads * 2 * 8 * 9 + P * w.num_kv_heads * 128 * 2  # NVFP4 in + FP8 out

    def roof(bound, achieved, peak, unit):
        return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4)}

    return {"quantize_chunk_ms": round(q_ms, 5), "quantize_chunk_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "quantize_chunk_bytes": q_bytes, "dequant_prefix_ms": round(d_ms, 5),
            "dequant_prefix_GBps": round(d_bytes / (d_ms * 1e-3) / 1e9, 1), "dequant_prefix_bytes": d_bytes,
            "dequant_prefix_fp8_ms": round(d8_ms, 5), "dequant_prefix_fp8_GBps": round(d8_bytes / (d8_ms * 1e-3) / 1e9, 1),
            "dequant_prefix_fp8_bytes": d8_bytes,
            "attn_ms": round(a_ms, 4), "attn_TFLOPs": round(a_flops / (a_ms * 1e-3) / 1e12, 1),
            "attn_fp8_ms": round(a8_ms, 4), "attn_fp8_TFLOPs": round(a_flops / (a8_ms * 1e-3) / 1e12, 1),
            "attn_flops": a_flops,
            "dequant_prefix_tiled_ms": round(dt_ms, 5), "attn_tiled_ms": round(at_ms, 4),
            "attn_tiled_TFLOPs": round(a_flops / (at_ms * 1e-3) / 1e12, 1),
            "attn_tiled_roofline": roof("mfma", a_flops / (at_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"),
            "step_tiled_ms": round(q_ms + dt_ms + at_ms, 4),
            "attn_roofline": roof("mfma", a_flops / (a_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"),
            "quantize_roofline": roof("hbm", q_bytes / (q_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "dequant_roofline": roof("hbm", d_bytes / (d_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
            "attn_fused_write_ms": round(af_ms, 4),
            "step_ms": round(q_ms + d_ms + a_ms, 4), "step_fp8_ms": round(q_ms + d8_ms + a8_ms, 4),
            "step_fused_ms": round(d_ms + af_ms, 4),
            "chunk_tokens": C, "prefix_tokens": P,
            "launches_timed": {"quantize_and_dequant": n_small, "attention": n_att},
            "note": "each kernel timed over back-to-back launches with events only around the loop; two different "
                    "prefixes alternate in the dequant, so no launch reads the previous one's bytes from the "
                    "last-level cache; step_fused_ms is the production prefill form (dequant, then the attention "
                    "launch that also quantize-writes the chunk)"}


def fill_pool_rows(w, pool, B, W, torch, row, n_tokens, step=65536):
    for t0 in range(0, n_tokens, step):
        t1 = min(n_tokens, t0 + step)
        k, v = W.kv(w, row, t0, t1, device="cuda")
        B.nvfp4_kv_quantize(k, v, torch.as_tensor(W.slots(w, row, t0, t1), device="cuda"), pool)
    torch.cuda.synchronize()


def measure(w, splits, B, W, torch, steps, warmup, fp8=True, keep_pool=False):
    """Every figure of one workload: the NVFP4 decode step (fused and three-launch),
    its split kernel with the HBM roofline, and the FP8 row at the same batch."""
    t_fill = time.perf_counter()
    pool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda")
    fill_pool(w, pool, B, W, torch)
    t_fill = time.perf_counter() - t_fill
    t = decode_step(w, pool, splits, B, W, torch, steps, warmup)
    kv_bytes = w.kv_bytes_per_step()
    gbs = kv_bytes / (t["ms"] * 1e-3) / 1e9
    k_gbs = kv_bytes / (t["k_ms"] * 1e-3) / 1e9
    ragged = len(set(w.seq_lens.tolist())) > 1
    r = {
        "batch": w.batch,
        "seq_len": f"U[{int(w.seq_lens.min())},{int(w.seq_lens.max())}]" if ragged else int(w.seq_lens[0]),
        "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "num_splits": splits,
        "kv_bytes_per_step": kv_bytes,
        "ms_per_step": round(t["ms"], 5),
        "GBps": round(gbs, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "decode_steps_per_s_per_layer": round(1e3 / t["ms"], 2),
        "tokens_per_s_per_layer": round(w.batch * 1e3 / t["ms"], 1),
        "roofline": {"bound": "hbm", "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": committed_traffic(w.name, splits),
                     "kernel": "k_decode_split", "kernel_ms": round(t["k_ms"], 5), "bytes_per_launch": kv_bytes},
        "step_three_launch_ms": round(t["ms_three"], 5),
        "wall_s_timed": round(t["wall"], 3),
        "pool_fill_s": round(t_fill, 2),
    }
    if fp8:
        pool_bytes = pool.data.numel()
        if not keep_pool:
            del pool
            torch.cuda.empty_cache()
        # the FP8 pool is 1.78x the NVFP4 one; both fit the 288 GB of HBM
        r["fp8_baseline"] = fp8_row(w, splits, B, W, torch, steps, warmup, t["ms"], t["k_ms"])
        r["fp8_baseline"]["nvfp4_pool_bytes"] = pool_bytes
        if not keep_pool:
            return r, None
    return r, pool


def capacity(B, W, torch, steps, warmup, rows_by_len):
    """The pages' capacity-driven comparison on this kernel pair: at each context
    length, FP8 at the resident count the pages report for an FP8 cache, NVFP4 at
    the count they report for NVFP4 (44 -> 70 at 32K, 10 -> 15 at 160K, 1 -> 2 at
    1M). Decode tokens/s per layer of each and their ratio. A row already measured
    in this run (a workload of the same batch and length) is reused."""
    out = []
    for L, b8, b4 in CAPACITY:
        row = {"seq_len": L, "fp8_batch": b8, "nvfp4_batch": b4}
        for fmt, b in (("fp8", b8), ("nvfp4", b4)):
            got = rows_by_len.get((fmt, b, L))
            if got is None:
                w = W.make_workload(f"capacity_{fmt}_{L}_b{b}", 2000 + b + L % 997, b, 64, 8, L)
                s = B.nvfp4_paged_decode_attn_default_splits(b, 8, L) if fmt == "nvfp4" else \
                    B.fp8_paged_decode_attn_default_splits(b, 8, L)
                if fmt == "fp8":
                    got = fp8_row(w, s, B, W, torch, steps, warmup)
                else:
                    got, _ = measure(w, s, B, W, torch, steps, warmup, fp8=False)
                torch.cuda.empty_cache()
            row[f"{fmt}_ms_per_step"] = got["ms_per_step"]
            row[f"{fmt}_tokens_per_s_per_layer"] = got["tokens_per_s_per_layer"]
            row[f"{fmt}_kv_bytes_per_step"] = got["kv_bytes_per_step"]
            row[f"{fmt}_kernel_frac"] = got["kernel_frac"] if fmt == "fp8" else got["roofline"]["frac"]
        row["nvfp4_over_fp8_tokens_per_s"] = round(row["nvfp4_tokens_per_s_per_layer"] /
                                                   row["fp8_tokens_per_s_per_layer"], 3)
        row["pages_peak_batch_gain_context"] = CAPACITY_PAGES_GAIN[L]
        out.append(row)
    return out


def main(argv=None):
    args = parse(argv)
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_skip, args.trace_steps, args.trace_warmup)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_bytes:
        copy_calibration(args.copy_bytes, args.steps)
        return
    import torch

    from bit_paged_kv_nvfp4_amd import binding as B
    from bit_paged_kv_nvfp4_amd import workload as W

    B.lib()  # fails loudly when the HIP library is missing
    torch.cuda.init()
    t_all = time.perf_counter()

    def splits_of(w):
        s = w.num_splits if args.splits < 0 else args.splits
        return s if s else B.nvfp4_paged_decode_attn_default_splits(w.batch, w.num_kv_heads, w.max_seq_len)

    fp8 = not args.no_fp8_baseline
    w = W.config(args.config)
    head, pool = measure(w, splits_of(w), B, W, torch, args.steps, args.warmup, fp8=fp8,
                         keep_pool=bool(w.extend_prefix))
    rows_by_len = {}

    def note_rows(wl, r):
        if len(set(wl.seq_lens.tolist())) == 1:
            L = int(wl.seq_lens[0])
            rows_by_len[("nvfp4", wl.batch, L)] = r
            if "fp8_baseline" in r:
                rows_by_len[("fp8", wl.batch, L)] = r["fp8_baseline"]

    note_rows(w, head)
    if w.extend_prefix:
        head["extend"] = extend_step(w, pool, B, W, torch, max(3, args.steps // 5), 2)
    del pool
    torch.cuda.empty_cache()
    workloads = {w.name: head}
    for c in [int(x) for x in args.workloads.split(",") if x.strip()]:
        if c == args.config:
            continue
        wc = W.config(c)
        r, p = measure(wc, splits_of(wc), B, W, torch, args.steps, args.warmup, fp8=fp8,
                       keep_pool=bool(wc.extend_prefix))
        if wc.extend_prefix:
            r["extend"] = extend_step(wc, p, B, W, torch, max(3, args.steps // 5), 2)
        del p
        torch.cuda.empty_cache()
        note_rows(wc, r)
        workloads[wc.name] = r
    res = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) Q/K/V, 4 K channels x8 per KV head, shuffled pages)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": head["seq_len"],
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": 128, "page_size": 16,
                   "num_splits": head["num_splits"], "kv_bytes_per_step": head["kv_bytes_per_step"]},
        "hbm_frac": head["hbm_frac"],
        "decode_steps_per_s_per_layer": head["decode_steps_per_s_per_layer"],
        "tokens_per_s_per_layer": head["tokens_per_s_per_layer"],
        "roofline": head["roofline"],
        "step_three_launch_ms": head["step_three_launch_ms"],
        "wall_s_timed": head["wall_s_timed"],
    }
    if "fp8_baseline" in head:
        res["fp8_baseline"] = head["fp8_baseline"]
    if "extend" in head:
        res["extend"] = head["extend"]
    if fp8 and not args.no_capacity:
        res["capacity"] = capacity(B, W, torch, args.steps, args.warmup, rows_by_len)
    res["workloads"] = {k: v for k, v in workloads.items() if k != w.name}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens, W, torch)
        w5 = W.config(5)
        if w5.name in workloads:
            res["cpu_baseline_extend"] = cpu_extend_baseline(w5, W, torch)
    res["bench_wall_s"] = round(time.perf_counter() - t_all, 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
