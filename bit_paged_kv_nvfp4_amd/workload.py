"""Seeded synthetic inputs for NVFP4 paged decode attention.

This module only draws random numbers and builds index tables. It holds none of
the method's arithmetic (no quantization, no attention) and is the one piece of
code that both the GPU path and the CPU oracle consume.

Workloads stand in for the serving runs that the pages measure (Qwen-family
models at 32K, 160K and 1M input tokens on one GPU) with the Llama-3.3-70B
attention geometry that page "NVFP4-KV-Cache auf der NVIDIA RTX PRO 6000
Blackwell Server Edition" uses for its byte arithmetic (section "Bytes pro
Token": 8 KV heads, head dimension 128) and the resident request counts of page
"SGLang stores KV cache in 4 bits ..." (section "Interpretation": 44 and 70 at
32K, 15 at 160K, 2 at 1M).

Recipe (all draws seeded):
  * Q: bfloat16 rounding of N(0, 1), shape [B, Hq, 128].
  * K, V: float32 N(0, 1), shape [tokens, Hkv, 128]; in K only, 4 of the 128
    channels of every KV head (drawn once per workload) are multiplied by 8.
    Values are drawn in fixed 4096-token chunks, each from its own generator
    seeded by (workload seed, sequence, chunk), so any chunk can be regenerated
    on its own.
  * Page table: a random permutation of all physical pages of the pool, handed
    out in order of (sequence, logical page); row stride = most pages of any
    sequence. Unused table entries are -1.
  * Sequence lengths: fixed, or integer-uniform on an inclusive range.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 128
PAGE_SIZE = 16
CHUNK_TOKENS = 4096
OUTLIER_CHANNELS = 4
OUTLIER_FACTOR = 8.0


def _mix(*vals: int) -> int:
    """splitmix64-style integer mixing of the seed tuple (63-bit result)."""
    x = 0x9E3779B97F4A7C15
    mask = (1 << 64) - 1
    for v in vals:
        x = (x ^ (int(v) & mask)) & mask
        x = (x + 0x9E3779B97F4A7C15) & mask
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        x = z ^ (z >> 31)
    return x & ((1 << 63) - 1)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: np.ndarray          # int32 [B] decode sequences
    page_table: np.ndarray        # int32 [B_all, stride]; rows >= B belong to the extend request
    num_pages: int
    outlier_channels: np.ndarray  # int64 [Hkv, 4]
    num_splits: int = 0           # 0 = library default
    extend_prefix: int = 0        # tokens of cached prefix of the extend request (0 = none)
    extend_chunk: int = 0         # tokens of the new bf16 chunk of the extend request
    description: str = ""

    @property
    def batch(self) -> int:
        return int(len(self.seq_lens))

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0

    @property
    def extend_row(self) -> int:
        """Page-table row of the extend request."""
        return self.batch

    def kv_bytes_per_step(self) -> int:
        """Algorithmic NVFP4 K+V bytes one decode step reads: 9 bytes per 16
        values (8 code bytes + 1 scale byte), K and V, every KV head."""
        tokens = int(self.seq_lens.astype(np.int64).sum())
        return tokens * self.num_kv_heads * 2 * (HEAD_DIM // 16) * 9


def _page_table(seed: int, pages_per_seq: list[int], extra_pages: int = 0):
    total = int(sum(pages_per_seq))
    g = torch.Generator(device="cpu").manual_seed(_mix(seed, 0xBA6E))
    perm = torch.randperm(total, generator=g).to(torch.int32).numpy()
    stride = max(pages_per_seq) if pages_per_seq else 1
    pt = np.full((len(pages_per_seq), stride), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per_seq):
        pt[b, :n] = perm[pos:pos + n]
        pos += n
    return pt, total


def _outliers(seed: int, num_kv_heads: int) -> np.ndarray:
    g = torch.Generator(device="cpu").manual_seed(_mix(seed, 0x0717))
    rows = [torch.randperm(HEAD_DIM, generator=g)[:OUTLIER_CHANNELS].sort().values for _ in range(num_kv_heads)]
    return torch.stack(rows).numpy().astype(np.int64)


def make_workload(name: str, seed: int, batch: int, num_q_heads: int, num_kv_heads: int,
                  seq_len: int | tuple[int, int], num_splits: int = 0, extend_prefix: int = 0,
                  extend_chunk: int = 0, description: str = "") -> Workload:
    if isinstance(seq_len, tuple):
        lo, hi = seq_len
        g = torch.Generator(device="cpu").manual_seed(_mix(seed, 0x5E0))
        lens = torch.randint(lo, hi + 1, (batch,), generator=g).to(torch.int32).numpy()
    else:
        lens = np.full(batch, seq_len, dtype=np.int32)
    pages = [int(-(-int(L) // PAGE_SIZE)) for L in lens]
    if extend_prefix or extend_chunk:
        pages.append(-(-(extend_prefix + extend_chunk) // PAGE_SIZE))
    pt, total = _page_table(seed, pages)
    return Workload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, seq_lens=lens,
                    page_table=pt, num_pages=total, outlier_channels=_outliers(seed, num_kv_heads),
                    num_splits=num_splits, extend_prefix=extend_prefix, extend_chunk=extend_chunk,
                    description=description)


def config(idx: int) -> Workload:
    """The five named workloads (1-based index)."""
    if idx == 1:
        return make_workload("tiny_b1_gqa8_2k", 1001, 1, 8, 1, 2048,
                             description="1 layer, batch 1, 8 query / 1 KV head, 2048 tokens")
    if idx == 2:
        return make_workload("llama70b_layer_32k_b44", 1002, 44, 64, 8, 32768,
                             description="Llama-3.3-70B layer shape, batch 44 x 32768 tokens")
    if idx == 3:
        return make_workload("llama70b_layer_32k_b70_ragged", 1003, 70, 64, 8, (24576, 32768),
                             description="Llama-3.3-70B layer shape, batch 70, lengths U[24576, 32768]")
    if idx == 4:
        return make_workload("long_160k_b15", 1004, 15, 64, 8, 163840, num_splits=64,
                             description="batch 15 x 163840 tokens, 64 splits")
    if idx == 5:
        return make_workload("extreme_1m_b2_extend", 1005, 2, 64, 8, 1048576, extend_prefix=163840,
                             extend_chunk=8192,
                             description="batch 2 x 1048576 tokens + extend request (163840-token prefix, "
                                         "8192-token bf16 chunk)")
    raise ValueError(idx)


def small_workload(seed: int, batch: int, num_q_heads: int, num_kv_heads: int, seq_lens, num_splits: int = 0,
                   name: str = "small") -> Workload:
    """Workload with explicit per-sequence lengths (for parity and edge tests)."""
    lens = np.asarray(seq_lens, dtype=np.int32)
    pages = [max(1, int(-(-int(L) // PAGE_SIZE))) for L in lens]
    pt, total = _page_table(seed, pages)
    return Workload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, seq_lens=lens,
                    page_table=pt, num_pages=total, outlier_channels=_outliers(seed, num_kv_heads),
                    num_splits=num_splits)


# ---- value draws ------------------------------------------------------------
def query(w: Workload, device: str | torch.device = "cpu") -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(_mix(w.seed, 0x9))
    q = torch.randn((w.batch, w.num_q_heads, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def extend_query(w: Workload, device: str | torch.device = "cpu") -> torch.Tensor:
    """Queries of the extend request's chunk: bfloat16 [chunk, Hq, 128]."""
    g = torch.Generator(device=device).manual_seed(_mix(w.seed, 0xE9))
    q = torch.randn((w.extend_chunk, w.num_q_heads, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def extend_inputs(seed: int, prefix_len: int, chunk_len: int, num_q_heads: int, num_kv_heads: int,
                  prefix_dtype=torch.bfloat16, device: str | torch.device = "cpu"):
    """Seeded inputs of one extend-attention call: q [C, Hq, 128] bf16; a prefix
    workspace K, V [P, Hkv, 128] in prefix_dtype (bfloat16 or float8_e4m3fn, cast
    from the same draws as a sequence's K/V, outlier channels included); chunk K, V
    [C, Hkv, 128] bf16 (the tokens that follow the prefix)."""
    w = small_workload(seed, 1, num_q_heads, num_kv_heads, [prefix_len + chunk_len])
    g = torch.Generator(device=device).manual_seed(_mix(seed, 0xE9))
    q = torch.randn((chunk_len, num_q_heads, HEAD_DIM), generator=g, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    k, v = kv(w, 0, 0, prefix_len + chunk_len, device)
    return (q, k[:prefix_len].to(prefix_dtype), v[:prefix_len].to(prefix_dtype), k[prefix_len:].to(torch.bfloat16),
            v[prefix_len:].to(torch.bfloat16))


def _kv_chunk(w: Workload, seq: int, chunk: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    g = torch.Generator(device=device).manual_seed(_mix(w.seed, 0xC4, seq, chunk))
    shape = (CHUNK_TOKENS, w.num_kv_heads, HEAD_DIM)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    oc = torch.as_tensor(w.outlier_channels, device=device)
    heads = torch.arange(w.num_kv_heads, device=device).unsqueeze(1).expand_as(oc)
    k[:, heads, oc] *= OUTLIER_FACTOR
    return k, v


def kv(w: Workload, seq: int, t0: int, t1: int, device: str | torch.device = "cpu"):
    """float32 K, V [t1 - t0, Hkv, 128] of tokens [t0, t1) of sequence ``seq``
    (``seq == w.batch`` is the extend request)."""
    ks, vs = [], []
    c0, c1 = t0 // CHUNK_TOKENS, (t1 - 1) // CHUNK_TOKENS
    for c in range(c0, c1 + 1):
        k, v = _kv_chunk(w, seq, c, device)
        a = max(t0, c * CHUNK_TOKENS) - c * CHUNK_TOKENS
        b = min(t1, (c + 1) * CHUNK_TOKENS) - c * CHUNK_TOKENS
        ks.append(k[a:b])
        vs.append(v[a:b])
    return torch.cat(ks), torch.cat(vs)


def extend_chunk_kv(w: Workload, device: str | torch.device = "cpu"):
    """The extend request's new chunk as bfloat16 [chunk, Hkv, 128] K, V (tokens
    [prefix, prefix + chunk) of that request)."""
    k, v = kv(w, w.extend_row, w.extend_prefix, w.extend_prefix + w.extend_chunk, device)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def slots(w: Workload, seq: int, t0: int, t1: int) -> np.ndarray:
    """slot = physical page * 16 + row of tokens [t0, t1) of sequence ``seq``."""
    t = np.arange(t0, t1, dtype=np.int64)
    pages = w.page_table[seq, t // PAGE_SIZE].astype(np.int64)
    return (pages * PAGE_SIZE + t % PAGE_SIZE).astype(np.int32)
