"""Parity at the five workloads' full sizes, in the launch configuration bench.py
times (same split rule). The GPU fills the whole pool and decodes the whole batch;
the oracle recomputes (sequence, KV head) pairs on its own: it quantizes the
same seeded K/V (bytes must match the GPU pool exactly) and evaluates fp64
attention for those heads' query heads (outputs within 2e-3 + 1e-2 |ref|). The
pairs: every KV head of the longest sequence (each of its segments is cut by
many workgroup windows, so window starts inside a segment and the merged runs
that close them are all in the check), and one head each of the first, last,
shortest and a random sequence. Every output and LSE of the batch must be
finite. Workload 5 also checks the extend
path: the 8192-token bf16 chunk's quantized bytes in full and sampled rows of the
dequantized 163840-token prefix, bit-exact."""
import os

import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import assert_close, bf16_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
CHUNK = 65536


def fill(w, pool, seqs):
    for b in seqs:
        L = int(w.seq_lens[b]) if b < w.batch else w.extend_prefix
        for t0 in range(0, L, CHUNK):
            t1 = min(L, t0 + CHUNK)
            k, v = W.kv(w, b, t0, t1, device="cuda")
            B.nvfp4_kv_quantize(k, v, torch.as_tensor(W.slots(w, b, t0, t1), device="cuda"), pool)
    torch.cuda.synchronize()


def oracle_head_pools(w, b, L, heads):
    """The oracle's own single-head pools of sequence b, one per listed KV head
    (same page ids); the K/V draws are made once."""
    pools = {h: np.zeros(oracle.pool_bytes(w.num_pages, 1), dtype=np.uint8) for h in heads}
    for t0 in range(0, L, CHUNK):
        t1 = min(L, t0 + CHUNK)
        k, v = W.kv(w, b, t0, t1, device="cuda")
        k, v = k.cpu().numpy(), v.cpu().numpy()
        for h in heads:
            oracle.quantize_to_pool(np.ascontiguousarray(k[:, h:h + 1]), np.ascontiguousarray(v[:, h:h + 1]),
                                    W.slots(w, b, t0, t1), w.num_pages, pool=pools[h], n_threads=THREADS)
        del k, v
    return pools


def gpu_slabs(w, gpool, pages, h):
    """GPU K and V slabs of head h for the given physical pages, as [n, 2304]."""
    data = gpool.data.view(w.num_pages, w.num_kv_heads, 2 * 1152)
    return data[torch.as_tensor(pages, device="cuda", dtype=torch.long), h].cpu().numpy()


def plan(w):
    """(sequence, KV heads) to check: every head of the longest sequence, one
    head each of the first, last, shortest and a random one."""
    rng = np.random.default_rng(w.seed)
    lens = w.seq_lens
    longest = int(np.argmax(lens))
    out = [(longest, list(range(w.num_kv_heads)))]
    for b in sorted({0, w.batch - 1, int(np.argmin(lens)), int(rng.integers(0, w.batch))} - {longest}):
        out.append((b, [int(rng.integers(0, w.num_kv_heads))]))
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_workload(cfg):
    w = W.config(cfg)
    print(f"workload {cfg} {w.name}: batch {w.batch}, pages {w.num_pages}", flush=True)
    splits = w.num_splits or B.nvfp4_paged_decode_attn_default_splits(w.batch, w.num_kv_heads, w.max_seq_len)
    gpool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda")
    fill(w, gpool, range(w.batch))
    q = W.query(w, device="cuda")
    pt = torch.as_tensor(w.page_table[:w.batch], device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    out = B.nvfp4_paged_decode_attn(q, pt, sl, gpool, w.sm_scale, w.max_seq_len, num_splits=splits,
                                    out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qbits = bf16_bits(q.cpu())
    group = w.num_q_heads // w.num_kv_heads
    pairs = 0
    for b, heads in plan(w):
        L = int(w.seq_lens[b])
        print(f"  seq {b} (len {L}) KV heads {heads}", flush=True)
        pools = oracle_head_pools(w, b, L, heads)
        pages = w.page_table[b, :(L + 15) // 16]
        for h in heads:
            got = gpu_slabs(w, gpool, pages, h)
            want = pools[h].reshape(w.num_pages, 2 * 1152)[pages]
            assert np.array_equal(got, want), f"seq {b} head {h}: {int((got != want).sum())} pool bytes differ"
            # the oracle's single-head view: query heads of KV head h become heads 0..group-1
            qh = np.ascontiguousarray(qbits[b:b + 1, h * group:(h + 1) * group])
            ref, ref_lse = oracle.decode_attn(qh, w.page_table[b:b + 1], w.seq_lens[b:b + 1], pools[h], 1,
                                              w.sm_scale, n_threads=THREADS)
            err = assert_close(out[b, h * group:(h + 1) * group], ref[0], what=f"cfg {cfg} seq {b} head {h}")
            assert_close(lse[b, h * group:(h + 1) * group], ref_lse[0], atol=1e-3, rtol=1e-4, what="lse")
            print(f"    head {h}: max abs err {err:.2e}", flush=True)
        del pools
        pairs += len(heads)
    print(f"  {pairs} of {w.batch * w.num_kv_heads} (sequence, KV head) pairs checked", flush=True)
    if w.extend_prefix:
        extend_checks(w, gpool)


def extend_checks(w, gpool):
    row, P, C = w.extend_row, w.extend_prefix, w.extend_chunk
    fill(w, gpool, [row])  # the cached prefix
    kc, vc = W.extend_chunk_kv(w, device="cuda")
    cslots = W.slots(w, row, P, P + C)
    B.nvfp4_kv_quantize(kc, vc, torch.as_tensor(cslots, device="cuda"), gpool)
    torch.cuda.synchronize()
    opool = oracle.quantize_to_pool(bf16_bits(kc.cpu()), bf16_bits(vc.cpu()), cslots, w.num_pages,
                                    pool=np.zeros(oracle.pool_bytes(w.num_pages, w.num_kv_heads), np.uint8),
                                    n_threads=THREADS)
    pages = np.unique(cslots // 16)
    got = gpool.data.view(w.num_pages, -1)[torch.as_tensor(pages, device="cuda", dtype=torch.long)].cpu().numpy()
    assert np.array_equal(got, opool.reshape(w.num_pages, -1)[pages]), "extend chunk bytes differ"
    print("  extend chunk quantize bit-exact", flush=True)
    # dequantize the prefix into a bf16 workspace; check sampled rows of every head
    k_ws = torch.empty((P, w.num_kv_heads, 128), dtype=torch.bfloat16, device="cuda")
    v_ws = torch.empty_like(k_ws)
    B.nvfp4_kv_dequant_workspace(gpool, torch.as_tensor(w.page_table[row:row + 1], device="cuda").contiguous(),
                                 torch.tensor([P], dtype=torch.int32, device="cuda"),
                                 torch.zeros(1, dtype=torch.int64, device="cuda"), P, k_ws, v_ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, 15, 16, P - 1], rng.integers(0, P, 60)]))
    for t in rows:
        k, v = W.kv(w, row, int(t), int(t) + 1, device="cuda")
        pool1 = oracle.quantize_to_pool(k.cpu().numpy(), v.cpu().numpy(), np.array([t % 16], np.int32), 1)
        for h in range(w.num_kv_heads):
            for kind, ws in ((0, k_ws), (1, v_ws)):
                ref = oracle.dequant_row(pool1, 0, int(t % 16), h, kind, w.num_kv_heads)
                want = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16)
                assert torch.equal(ws[int(t), h].cpu().view(torch.int16), want), (t, h, kind)
    print(f"  extend prefix dequant bit-exact on {len(rows)} rows x {w.num_kv_heads} heads", flush=True)
