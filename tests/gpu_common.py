"""Shared helpers of the GPU parity tests: fill pools on both sides from the same
seeded inputs (the GPU through the library, the oracle on its own), compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W

ATOL = 2e-3
RTOL = 1e-2


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def gpu_pool_from_kv(w: W.Workload, kv_by_seq, g: float = 1.0) -> B.Pool:
    """kv_by_seq: list of (k, v) float32/bf16 [L, Hkv, 128] tensors (any device)."""
    pool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda", global_scale=g)
    for b, (k, v) in enumerate(kv_by_seq):
        L = k.shape[0]
        if L == 0:
            continue
        slots = torch.as_tensor(W.slots(w, b, 0, L), device="cuda")
        B.nvfp4_kv_quantize(k.cuda().contiguous(), v.cuda().contiguous(), slots, pool)
    torch.cuda.synchronize()
    return pool


def oracle_pool_from_kv(w: W.Workload, kv_by_seq, g: float = 1.0) -> np.ndarray:
    pool = np.zeros(oracle.pool_bytes(w.num_pages, w.num_kv_heads), dtype=np.uint8)
    for b, (k, v) in enumerate(kv_by_seq):
        L = k.shape[0]
        if L == 0:
            continue
        kk, vv = k.cpu(), v.cpu()
        if kk.dtype == torch.bfloat16:
            kn, vn = bf16_bits(kk), bf16_bits(vv)
        else:
            kn, vn = kk.numpy(), vv.numpy()
        oracle.quantize_to_pool(kn, vn, W.slots(w, b, 0, L), w.num_pages, g=g, pool=pool, n_threads=8)
    return pool


def run_decode(w: W.Workload, pool: B.Pool, q: torch.Tensor, num_splits: int = 0, out_dtype=torch.float32,
               page_table: np.ndarray | None = None, sm_scale: float | None = None):
    pt = torch.as_tensor(w.page_table if page_table is None else page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    out = B.nvfp4_paged_decode_attn(q.cuda().contiguous(), pt, sl, pool, w.sm_scale if sm_scale is None else sm_scale,
                                    max(1, w.max_seq_len), num_splits=num_splits, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def assert_close(gpu: np.ndarray, ref: np.ndarray, atol=ATOL, rtol=RTOL, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), ref.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r}")
    return float(err.max())
