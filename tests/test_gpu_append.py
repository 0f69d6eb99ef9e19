"""GPU parity of the fused decode step (nvfp4_paged_decode_attn_append and
fp8_paged_decode_attn_append, through the C ABI): the launch writes each
sequence's newest token into the pool and attends over the updated cache.

The GPU pool holds tokens 0..L-2 of each sequence and, at the newest token's
slot, a different token's bytes (so the fused write must replace them and leave
the row that shares its V bytes alone). The oracle quantizes all L tokens into
a zeroed pool on its own. Bars: pool bytes bit-exact; attention
|gpu - ref| <= 2e-3 + 1e-2 |ref|, lse within 1e-3 + 1e-4 |ref|."""
import os

import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import assert_close, bf16_bits

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _np(t):
    t = t.cpu()
    return bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()


def _setup(w, fp8, dt, g=1.0, ks=1.0, vs=1.0):
    """GPU pool with every token but the newest (whose slot holds another token's
    bytes), the oracle pool with all tokens, and the newest rows [B, Hkv, 128]."""
    hkv = w.num_kv_heads
    if fp8:
        gpool = B.Fp8Pool(w.num_pages, hkv, device="cuda", k_scale=ks, v_scale=vs)
        opool = np.zeros(oracle.fp8_pool_bytes(w.num_pages, hkv), dtype=np.uint8)
        quant = B.fp8_kv_quantize
    else:
        gpool = B.Pool(w.num_pages, hkv, device="cuda", global_scale=g)
        opool = np.zeros(oracle.pool_bytes(w.num_pages, hkv), dtype=np.uint8)
        quant = B.nvfp4_kv_quantize
    k_new = torch.zeros((w.batch, hkv, 128), dtype=dt)
    v_new = torch.zeros_like(k_new)
    for b, L in enumerate(w.seq_lens):
        L = int(L)
        if L == 0:
            continue
        k, v = (x.to(dt) for x in W.kv(w, b, 0, L))
        slots = W.slots(w, b, 0, L)
        if L > 1:
            quant(k[:-1].cuda().contiguous(), v[:-1].cuda().contiguous(),
                  torch.as_tensor(slots[:-1], device="cuda"), gpool)
        # stale bytes at the newest slot: token 0's rows scaled, written alone
        quant((k[:1] * 3).cuda().contiguous(), (v[:1] * -2).cuda().contiguous(),
              torch.as_tensor(slots[-1:], device="cuda"), gpool)
        k_new[b], v_new[b] = k[-1], v[-1]
        if fp8:
            oracle.fp8_quantize_to_pool(_np(k), _np(v), slots, w.num_pages, ks, vs, pool=opool)
        else:
            oracle.quantize_to_pool(_np(k), _np(v), slots, w.num_pages, g=g, pool=opool, n_threads=THREADS)
    torch.cuda.synchronize()
    return gpool, opool, k_new, v_new


def _append(w, fp8, gpool, q, k_new, v_new, splits):
    pt = torch.as_tensor(w.page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    fn = B.fp8_paged_decode_attn_append if fp8 else B.nvfp4_paged_decode_attn_append
    out = fn(q.cuda().contiguous(), k_new.cuda(), v_new.cuda(), pt, sl, gpool, w.sm_scale, max(1, w.max_seq_len),
             num_splits=splits, out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, Hq, Hkv, lengths, splits, dtype of the new rows, global scale
    ("ragged_tails", 8, 2, [1, 2, 3, 4, 5, 15, 16, 17, 33, 100], 3, torch.float32, 1.0),
    ("llama_shape_bf16", 64, 8, [300, 1000, 1], 0, torch.bfloat16, 1.0),
    ("many_splits", 16, 1, [4096, 37], 64, torch.float32, 1.0),
    ("group3_g_half", 12, 4, [65, 2, 0, 48], 0, torch.float32, 0.5),
    ("one_split", 8, 8, [31, 18], 1, torch.bfloat16, 1.0),
]


@pytest.mark.parametrize("fp8", [False, True], ids=["nvfp4", "fp8"])
@pytest.mark.parametrize("name,hq,hkv,lens,splits,dt,g", CASES, ids=[c[0] for c in CASES])
def test_append_matches_oracle(name, hq, hkv, lens, splits, dt, g, fp8):
    print(f"case {name} {'fp8' if fp8 else 'nvfp4'}: Hq={hq} Hkv={hkv} lens={lens} splits={splits}", flush=True)
    w = W.small_workload(900 + len(name), len(lens), hq, hkv, lens, num_splits=splits, name=name)
    ks, vs = (0.5, 2.0) if fp8 and g != 1.0 else (1.0, 1.0)
    gpool, opool, k_new, v_new = _setup(w, fp8, dt, g=g, ks=ks, vs=vs)
    q = W.query(w)
    out, lse = _append(w, fp8, gpool, q, k_new, v_new, splits)
    gbytes = gpool.data.cpu().numpy()
    assert np.array_equal(gbytes, opool), f"pool bytes differ at {np.flatnonzero(gbytes != opool)[:8]}"
    if fp8:
        ref, ref_lse = oracle.fp8_decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale, ks, vs,
                                              n_threads=THREADS)
    else:
        ref, ref_lse = oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale, g=g,
                                          n_threads=THREADS)
    live = np.asarray(w.seq_lens) > 0
    err = assert_close(out[live], ref[live], what=name)
    assert_close(lse[live], ref_lse[live], atol=1e-3, rtol=1e-4, what=name + " lse")
    assert np.all(out[~live] == 0) and np.all(np.isneginf(lse[~live]))
    print(f"  max abs err {err:.3e}", flush=True)


def test_append_twice_is_idempotent():
    """Appending the same rows again rewrites identical bytes and gives the same
    result (the benchmark's step does exactly this)."""
    w = W.small_workload(950, 3, 16, 2, [70, 16, 5], name="twice")
    gpool, opool, k_new, v_new = _setup(w, False, torch.bfloat16)
    q = W.query(w)
    out1, lse1 = _append(w, False, gpool, q, k_new, v_new, 0)
    out2, lse2 = _append(w, False, gpool, q, k_new, v_new, 0)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
