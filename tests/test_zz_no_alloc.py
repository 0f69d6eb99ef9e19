"""GPU checks of nvfp4_paged_decode_attn_noalloc, the decode entry point for
callers that cannot allocate device memory: its split states live in the
library's fixed per-GPU scratch array. Same kernels as nvfp4_paged_decode_attn,
so with the same split count the outputs must be bit-identical to it, and within
the attention tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import assert_close, bf16_bits, gpu_pool_from_kv, oracle_pool_from_kv

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _setup(seed, batch, hq, hkv, lens):
    w = W.small_workload(seed, batch, hq, hkv, lens, name="noalloc")
    kv = [W.kv(w, b, 0, int(L)) if L else (torch.zeros((0, hkv, 128)), torch.zeros((0, hkv, 128)))
          for b, L in enumerate(w.seq_lens)]
    return w, kv, gpu_pool_from_kv(w, kv), W.query(w)


def _both(w, pool, q, splits):
    pt = torch.as_tensor(w.page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    qd = q.cuda().contiguous()
    lse_a = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    ref = B.nvfp4_paged_decode_attn(qd, pt, sl, pool, w.sm_scale, w.max_seq_len, num_splits=splits,
                                    out_dtype=torch.float32, lse=lse_a)
    got = B.nvfp4_paged_decode_attn_noalloc(qd, pt, sl, pool, w.sm_scale, w.max_seq_len,
                                            num_splits=0 if splits == 0 else splits, out_dtype=torch.float32,
                                            lse=lse_b)
    torch.cuda.synchronize()
    return ref, lse_a, got, lse_b


def test_noalloc_two_calls_second_smaller():
    print("noalloc: B3 [300, 47, 1000] then B2 [17, 5]", flush=True)
    for seed, batch, hq, hkv, lens in ((901, 3, 16, 2, [300, 47, 1000]), (902, 2, 8, 1, [17, 5])):
        w, kv, pool, q = _setup(seed, batch, hq, hkv, lens)
        for splits in (0, 3):
            ref, lse_a, got, lse_b = _both(w, pool, q, splits)
            assert torch.equal(got, ref), f"noalloc differs from the workspace call (splits {splits})"
            assert torch.equal(lse_b, lse_a)
        opool = oracle_pool_from_kv(w, kv)
        o_ref, o_lse = oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale,
                                          n_threads=8)
        assert_close(got.cpu().numpy(), o_ref, what=f"noalloc vs oracle {lens}")
        assert_close(lse_b.cpu().numpy(), o_lse, atol=1e-3, rtol=1e-4, what="noalloc lse vs oracle")


def test_noalloc_lowers_default_splits_to_fit_scratch():
    # 16 sequences x 16 query heads of one KV head at 65536 tokens: the default
    # split count's states exceed the 64 MiB scratch, so the call lowers it
    batch, hq, hkv, L = 16, 16, 1, 65536
    print(f"noalloc: B{batch} x {L}, group {hq}", flush=True)
    d = B.nvfp4_paged_decode_attn_default_splits(batch, hkv, L)
    assert B.nvfp4_paged_decode_attn_workspace_bytes(batch, hq, d) > SCRATCH
    fit = max(s for s in range(1, d + 1) if B.nvfp4_paged_decode_attn_workspace_bytes(batch, hq, s) <= SCRATCH)
    w = W.small_workload(903, batch, hq, hkv, [L] * batch, name="noalloc_big")
    pool = B.Pool(w.num_pages, hkv, device="cuda")
    for b in range(batch):
        k, v = W.kv(w, b, 0, L, device="cuda")
        B.nvfp4_kv_quantize(k, v, torch.as_tensor(W.slots(w, b, 0, L), device="cuda"), pool)
    q = W.query(w)
    pt = torch.as_tensor(w.page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    ref = B.nvfp4_paged_decode_attn(q.cuda(), pt, sl, pool, w.sm_scale, L, num_splits=fit, out_dtype=torch.float32)
    got = B.nvfp4_paged_decode_attn_noalloc(q.cuda(), pt, sl, pool, w.sm_scale, L, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "noalloc with the lowered default differs from the workspace call"
    # a sample of rows against the oracle over its own quantization of the same K/V
    seqs = [0, 7, 15]
    opool = np.zeros(oracle.pool_bytes(w.num_pages, hkv), dtype=np.uint8)
    for b in seqs:
        # the same draws as the device pool's (the CUDA generator, copied back)
        k, v = W.kv(w, b, 0, L, device="cuda")
        oracle.quantize_to_pool(k.cpu().numpy(), v.cpu().numpy(), W.slots(w, b, 0, L), w.num_pages, pool=opool,
                                n_threads=8)
    units = [b * hq + h for b in seqs for h in (0, 5, 15)]
    o_ref, _ = oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale, units=units,
                                  n_threads=8)
    g = got.cpu().numpy()
    for u in units:
        b, h = divmod(u, hq)
        assert_close(g[b, h], o_ref[b, h], what=f"noalloc big row ({b}, {h})")
    # and a smaller call right after, on the same scratch
    w2, kv2, pool2, q2 = _setup(904, 2, 16, 2, [33, 700])
    ref2, la, got2, lb = _both(w2, pool2, q2, 0)
    assert torch.equal(got2, ref2) and torch.equal(lb, la)
