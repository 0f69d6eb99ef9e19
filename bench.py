#!/usr/bin/env python3
"""Benchmark of NVFP4 paged decode attention on one MI355X.

One step = one decode step of one layer for the whole batch: the split-K decode
kernel plus the split combine, reading the batch's entire NVFP4 K/V cache.
Inputs (pool, Q, page table) are resident in HBM before the timed region; the
pool is filled once by the library's quantize-on-write kernel from seeded
synthetic K/V.

Prints one JSON line (rank 0, N = 1):
  value      KV-read GB/s = algorithmic NVFP4 KV bytes per step / time per step
  roofline   HBM roofline of the dominant kernel (decode split kernel), timed
             live with HIP events on the stream it runs on
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "NVFP4 paged decode-attn KV-read GB/s (% of HBM peak) + decode steps/s/layer"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (2 = batch 44 x 32K, the metric's workload)")
    ap.add_argument("--splits", type=int, default=-1, help="-1 = workload setting / library default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=2)
    return ap.parse_args()


def fill_pool(w, pool, B, W, torch):
    """Quantize-on-write every sequence's K/V into the pool (library kernel)."""
    step = 65536
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for t0 in range(0, L, step):
            t1 = min(L, t0 + step)
            k, v = W.kv(w, b, t0, t1, device="cuda")
            slots = torch.as_tensor(W.slots(w, b, t0, t1), device="cuda")
            B.nvfp4_kv_quantize(k, v, slots, pool)
    torch.cuda.synchronize()


def cpu_baseline(w, n_seqs, W, torch):
    """The oracle (fp64 attention over its own NVFP4 quantization of the same
    seeded K/V) on the first n_seqs sequences, all heads. Only the attention is
    timed; the sample's KV bytes over that time give a GB/s-equivalent."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    n_seqs = max(1, min(n_seqs, w.batch))
    lens = w.seq_lens[:n_seqs]
    sub = W.Workload(name=w.name, seed=w.seed, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                     seq_lens=lens, page_table=w.page_table[:n_seqs], num_pages=w.num_pages,
                     outlier_channels=w.outlier_channels)
    pool = np.zeros(oracle.pool_bytes(w.num_pages, w.num_kv_heads), dtype=np.uint8)
    for b in range(n_seqs):
        k, v = W.kv(w, b, 0, int(lens[b]), device="cuda")
        oracle.quantize_to_pool(k.cpu().numpy(), v.cpu().numpy(), W.slots(w, b, 0, int(lens[b])), w.num_pages,
                                pool=pool, n_threads=cores)
        del k, v
    q = W.query(w)[:n_seqs].contiguous().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    oracle.decode_attn(q, sub.page_table, lens, pool, w.num_kv_heads, w.sm_scale, n_threads=cores)
    dt = time.perf_counter() - t0
    kv_bytes = sub.kv_bytes_per_step()
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_seqs} of {w.batch} sequences x all {w.num_kv_heads} KV heads "
                      f"({int(lens.sum())} tokens, {kv_bytes} KV bytes), fp64 attention only, {dt:.2f} s",
            "seconds": round(dt, 3), "decode_steps_per_s_equiv": round(dt and (kv_bytes / w.kv_bytes_per_step()) / dt, 6)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_paged_kv_nvfp4_amd import binding as B
    from bit_paged_kv_nvfp4_amd import workload as W

    B.lib()  # fails loudly when the HIP library is missing
    torch.cuda.init()
    w = W.config(args.config)
    splits = w.num_splits if args.splits < 0 else args.splits
    if splits == 0:
        splits = B.nvfp4_paged_decode_attn_default_splits(w.batch, w.num_kv_heads, w.max_seq_len)
    t_fill = time.perf_counter()
    pool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda")
    fill_pool(w, pool, B, W, torch)
    t_fill = time.perf_counter() - t_fill
    q = W.query(w, device="cuda")
    pt = torch.as_tensor(w.page_table[:w.batch], device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    ws = torch.empty(B.nvfp4_paged_decode_attn_workspace_bytes(w.batch, w.num_q_heads, splits), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        B.nvfp4_paged_decode_attn(q, pt, sl, pool, w.sm_scale, w.max_seq_len, num_splits=splits, workspace=ws,
                                  out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    kv_bytes = w.kv_bytes_per_step()
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    steps_per_s = 1e3 / ms
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) Q/K/V, 4 K channels x8, shuffled pages)",
        "config": {"workload": w.name, "batch": w.batch, "seq_lens": "ragged" if len(set(w.seq_lens.tolist())) > 1
                   else int(w.seq_lens[0]), "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": 128, "page_size": 16, "num_splits": splits, "kv_bytes_per_step": kv_bytes},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "decode_steps_per_s_per_layer": round(steps_per_s, 2),
        "tokens_per_s_per_layer": round(steps_per_s * w.batch, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode step (split kernel + combine kernel), HIP events over the timed region"},
        "wall_s_timed": round(wall, 3),
        "pool_fill_s": round(t_fill, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_seqs, W, torch)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
