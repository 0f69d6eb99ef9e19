"""GPU checks of the global-scale calibration hook: nvfp4_kv_amax (through the
C ABI) equals the oracle's amax exactly, NaN elements ignored on both sides;
and a pool quantized at the calibrated g is bit-exact against the oracle's at
that g, with a smaller dequantization error than g = 1 on small values."""
import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import bf16_bits, gpu_pool_from_kv, oracle_pool_from_kv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T", [0, 1, 1000, 70000])
def test_amax_matches_oracle(dt, T):
    print(f"amax {dt} T={T}", flush=True)
    w = W.small_workload(90 + T % 7, 1, 8, 8, [max(T, 1)])
    k, v = W.kv(w, 0, 0, max(T, 1))
    k, v = k[:T].to(dt), (v[:T] * 3).to(dt)
    if T > 5:
        k[T // 2, 3, 17] = float("nan")
        v[T - 1, 7, 127] = -1e4
    out = B.nvfp4_kv_amax(k.cuda().contiguous(), v.cuda().contiguous())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if dt == torch.float32:
        ok, ov = k.numpy(), v.numpy()
    else:
        ok, ov = bf16_bits(k), bf16_bits(v)
    ref = [oracle.amax(ok), oracle.amax(ov)] if T else [0.0, 0.0]
    assert got[0] == ref[0] and got[1] == ref[1], (got, ref)


def test_calibrated_scale_end_to_end():
    """Small K/V values (x 1e-3): the calibrated g (a power of two) quantizes to the
    oracle's bytes at that g, and dequantizes closer to the inputs than g = 1."""
    lens = [70, 33]
    w = W.small_workload(95, len(lens), 16, 2, lens)
    kv = [tuple(x * 1e-3 for x in W.kv(w, b, 0, L)) for b, L in enumerate(lens)]
    am = max(float(B.nvfp4_kv_amax(k.cuda(), v.cuda()).max()) for k, v in kv)
    g = B.nvfp4kv_global_scale_for_amax(am)
    assert g == oracle.global_scale_for_amax(am) and g < 1.0
    errs = {}
    for gg in (g, 1.0):
        gpool = gpu_pool_from_kv(w, kv, g=gg)
        opool = oracle_pool_from_kv(w, kv, g=gg)
        assert np.array_equal(gpool.data.cpu().numpy(), opool), f"pool bytes differ at g={gg}"
        ko, vo = oracle.dequant_workspace(opool, w.num_kv_heads, w.page_table, w.seq_lens, g=gg)
        ref = np.concatenate([np.concatenate([k.numpy(), v.numpy()], axis=1) for k, v in kv])
        got = np.concatenate([ko, vo], axis=1)
        errs[gg] = float(np.sqrt(((got - ref) ** 2).sum() / (ref ** 2).sum()))
    print(f"  g={g}: rel-L2 {errs[g]:.4f}; g=1: {errs[1.0]:.4f}")
    assert errs[g] < errs[1.0]
