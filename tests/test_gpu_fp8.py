"""GPU parity of the FP8 E4M3 baseline (fp8_kv_quantize, fp8_paged_decode_attn,
through the C ABI) against the oracle's FP8 cache and decode attention.

Bars: pool bytes bit-exact; attention |gpu - ref| <= 2e-3 + 1e-2 |ref|, lse
within 1e-3 + 1e-4 |ref|."""
import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import assert_close, bf16_bits

pytestmark = pytest.mark.gpu


def _kv(w, dtype=torch.float32):
    return [tuple(x.to(dtype) for x in W.kv(w, b, 0, int(L))) for b, L in enumerate(w.seq_lens)]


def _pools(w, kv, ks, vs):
    gpool = B.Fp8Pool(w.num_pages, w.num_kv_heads, device="cuda", k_scale=ks, v_scale=vs)
    opool = np.zeros(oracle.fp8_pool_bytes(w.num_pages, w.num_kv_heads), dtype=np.uint8)
    for b, (k, v) in enumerate(kv):
        L = k.shape[0]
        if L == 0:
            continue
        slots = W.slots(w, b, 0, L)
        B.fp8_kv_quantize(k.cuda().contiguous(), v.cuda().contiguous(), torch.as_tensor(slots, device="cuda"), gpool)
        kk, vv = k.cpu(), v.cpu()
        kn, vn = (bf16_bits(kk), bf16_bits(vv)) if kk.dtype == torch.bfloat16 else (kk.numpy(), vv.numpy())
        oracle.fp8_quantize_to_pool(kn, vn, slots, w.num_pages, ks, vs, pool=opool)
    torch.cuda.synchronize()
    return gpool, opool


def _decode(w, gpool, q, splits=0, sm=None):
    pt = torch.as_tensor(w.page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    out = B.fp8_paged_decode_attn(q.cuda().contiguous(), pt, sl, gpool, w.sm_scale if sm is None else sm,
                                  max(1, w.max_seq_len), num_splits=splits, out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, Hq, Hkv, lengths, splits, k_scale, v_scale, source dtype
    ("ragged_tails", 8, 2, [1, 15, 16, 17, 33, 100], 3, 1.0, 1.0, torch.float32),
    ("llama_shape_bf16", 64, 8, [300, 1000], 0, 1.0, 1.0, torch.bfloat16),
    ("scales", 16, 2, [513, 64], 0, 0.5, 2.0, torch.float32),
    ("group1", 4, 4, [50], 2, 1.0, 1.0, torch.float32),
    ("group3", 12, 4, [65, 2], 0, 4.0, 0.25, torch.float32),
    ("group16_many_splits", 16, 1, [4096], 64, 1.0, 1.0, torch.float32),
    ("empty_and_single", 8, 1, [0, 1, 16], 0, 1.0, 1.0, torch.float32),
]


@pytest.mark.parametrize("name,hq,hkv,lens,splits,ks,vs,dt", CASES, ids=[c[0] for c in CASES])
def test_fp8_quantize_and_decode_match_oracle(name, hq, hkv, lens, splits, ks, vs, dt):
    print(f"case {name}: Hq={hq} Hkv={hkv} lens={lens} splits={splits} scales {ks}/{vs}", flush=True)
    w = W.small_workload(700 + len(name), len(lens), hq, hkv, lens, num_splits=splits, name=name)
    kv = [tuple(x.to(dt) for x in W.kv(w, b, 0, L)) if L > 0 else
          (torch.zeros((0, hkv, 128), dtype=dt), torch.zeros((0, hkv, 128), dtype=dt)) for b, L in enumerate(lens)]
    gpool, opool = _pools(w, kv, ks, vs)
    gbytes = gpool.data.cpu().numpy()
    assert np.array_equal(gbytes, opool), f"pool bytes differ at {np.flatnonzero(gbytes != opool)[:8]}"
    q = W.query(w)
    out, lse = _decode(w, gpool, q, splits)
    ref, ref_lse = oracle.fp8_decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale, ks, vs,
                                          n_threads=8)
    live = np.asarray(w.seq_lens) > 0
    err = assert_close(out[live], ref[live], what=name)
    assert_close(lse[live], ref_lse[live], atol=1e-3, rtol=1e-4, what=name + " lse")
    assert np.all(out[~live] == 0) and np.all(np.isneginf(lse[~live]))
    print(f"  max abs err {err:.3e}")


def test_fp8_full_size_sampled_rows():
    """The B44 x 32K workload in the launch configuration bench.py times (default
    splits); the oracle quantizes the sampled sequences' K/V itself and checks
    their attention rows."""
    w = W.config(2)
    print(f"full size {w.name}", flush=True)
    gpool = B.Fp8Pool(w.num_pages, w.num_kv_heads, device="cuda")
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for t0 in range(0, L, 65536):
            t1 = min(L, t0 + 65536)
            k, v = W.kv(w, b, t0, t1, device="cuda")
            B.fp8_kv_quantize(k, v, torch.as_tensor(W.slots(w, b, t0, t1), device="cuda"), gpool)
    q = W.query(w)
    out, lse = _decode(w, gpool, q)
    seqs = [0, 17, 43]
    opool = np.zeros(oracle.fp8_pool_bytes(w.num_pages, w.num_kv_heads), dtype=np.uint8)
    for b in seqs:
        # the same draws as the GPU fill (device generator), copied to the host
        L = int(w.seq_lens[b])
        k, v = W.kv(w, b, 0, L, device="cuda")
        oracle.fp8_quantize_to_pool(k.cpu().numpy(), v.cpu().numpy(), W.slots(w, b, 0, L), w.num_pages, pool=opool)
    units = [b * w.num_q_heads + h for b in seqs for h in (0, 9, 63)]
    ref, ref_lse = oracle.fp8_decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, w.num_kv_heads, w.sm_scale,
                                          units=units, n_threads=8)
    bi = np.array([u // w.num_q_heads for u in units])
    hi = np.array([u % w.num_q_heads for u in units])
    err = assert_close(out[bi, hi], ref[bi, hi], what="sampled rows")
    assert_close(lse[bi, hi], ref_lse[bi, hi], atol=1e-3, rtol=1e-4, what="sampled lse")
    print(f"  max abs err {err:.3e}")
