"""Pins of the oracle's extend attention (a chunk of queries over a dequantized
prefix workspace plus the chunk's own keys and values, causal over the chunk)
against torch's fp64 scaled_dot_product_attention with an explicit mask, and
against closed forms."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from tests.test_oracle_attention import bf16_bits

PRE_DTYPES = ["f32", "bf16", "fp8"]


def _bf16(rng, shape, scale=1.0):
    return torch.tensor(rng.standard_normal(shape) * scale, dtype=torch.float32).to(torch.bfloat16)


def _prefix(rng, P, hkv, kind):
    """(values fp64 [P, hkv, 128], the oracle's input array) for a workspace dtype."""
    if kind == "f32":
        x = rng.standard_normal((P, hkv, 128)).astype(np.float32)
        return x.astype(np.float64), x
    if kind == "bf16":
        t = _bf16(rng, (P, hkv, 128))
        return t.double().numpy(), bf16_bits(t)
    b = rng.integers(0, 256, size=(P, hkv, 128), dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    vals = torch.tensor(b).view(torch.float8_e4m3fn).double().numpy()
    return vals, b


def sdpa_extend_ref(q, kp, vp, kc, vc, hq, hkv, sm_scale):
    """Library reference: fp64 SDPA with KV heads repeated for GQA and a boolean
    mask that shows query i every prefix row and chunk rows 0..i."""
    C, P = q.shape[0], kp.shape[0]
    k = torch.cat([torch.as_tensor(kp), kc.double()]).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    v = torch.cat([torch.as_tensor(vp), vc.double()]).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    qq = q.double().permute(1, 0, 2)  # [Hq, C, D]
    col = torch.arange(P + C)
    mask = (col[None, :] < P) | (col[None, :] - P <= torch.arange(C)[:, None])
    o = F.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=sm_scale)
    s = (qq @ k.transpose(1, 2)) * sm_scale
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("kind", PRE_DTYPES)
@pytest.mark.parametrize("P,C,hq,hkv", [(37, 19, 8, 2), (0, 23, 4, 1), (5, 1, 16, 2)])
def test_extend_vs_library_sdpa(oracle_lib, kind, P, C, hq, hkv):
    rng = np.random.default_rng(31 + P + C)
    q = _bf16(rng, (C, hq, 128))
    kp, kp_in = _prefix(rng, P, hkv, kind)
    vp, vp_in = _prefix(rng, P, hkv, kind)
    kc, vc = _bf16(rng, (C, hkv, 128)), _bf16(rng, (C, hkv, 128))
    sm = 128 ** -0.5
    out, lse = oracle_lib.extend_attn(bf16_bits(q), kp_in, vp_in, bf16_bits(kc), bf16_bits(vc), sm)
    ref, ref_lse = sdpa_extend_ref(q, kp, vp, kc, vc, hq, hkv, sm)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_first_chunk_query_without_prefix_sees_only_itself(oracle_lib):
    rng = np.random.default_rng(41)
    C, hq, hkv = 6, 8, 2
    q, kc, vc = _bf16(rng, (C, hq, 128)), _bf16(rng, (C, hkv, 128)), _bf16(rng, (C, hkv, 128))
    empty = np.zeros((0, hkv, 128), dtype=np.uint16)
    out, lse = oracle_lib.extend_attn(bf16_bits(q), empty, empty, bf16_bits(kc), bf16_bits(vc), 0.125)
    for qh in range(hq):
        h = qh // (hq // hkv)
        assert np.array_equal(out[0, qh], vc[0, h].double().numpy())
        dot = float((q[0, qh].double() * kc[0, h].double()).sum())
        assert lse[0, qh] == pytest.approx(0.125 * dot, rel=1e-14, abs=1e-14)


def test_constant_keys_give_running_mean_of_values(oracle_lib):
    # every visible key equal: uniform weights, so query i returns the mean of the
    # P + i + 1 value rows it sees and lse = logit + ln(P + i + 1)
    rng = np.random.default_rng(42)
    P, C, hq, hkv = 11, 9, 8, 1
    key = _bf16(rng, (1, hkv, 128))
    kp_t = key.expand(P, hkv, 128).contiguous()
    kc = key.expand(C, hkv, 128).contiguous()
    vp_t, vc = _bf16(rng, (P, hkv, 128)), _bf16(rng, (C, hkv, 128))
    q = _bf16(rng, (C, hq, 128))
    out, lse = oracle_lib.extend_attn(bf16_bits(q), bf16_bits(kp_t), bf16_bits(vp_t), bf16_bits(kc), bf16_bits(vc),
                                      0.0625)
    vals = torch.cat([vp_t, vc]).double().numpy()[:, 0]
    for i in range(C):
        mean = vals[:P + i + 1].mean(axis=0)
        np.testing.assert_allclose(out[i], np.broadcast_to(mean, (hq, 128)), rtol=1e-13, atol=1e-13)
        logit = 0.0625 * (q[i].double() @ key[0, 0].double()).numpy()
        np.testing.assert_allclose(lse[i], logit + np.log(P + i + 1), rtol=1e-13, atol=1e-13)


def test_units_subset_and_threads_agree(oracle_lib):
    rng = np.random.default_rng(43)
    P, C, hq, hkv = 20, 12, 8, 2
    q = _bf16(rng, (C, hq, 128))
    kp, kp_in = _prefix(rng, P, hkv, "fp8")
    vp, vp_in = _prefix(rng, P, hkv, "fp8")
    kc, vc = _bf16(rng, (C, hkv, 128)), _bf16(rng, (C, hkv, 128))
    full, full_lse = oracle_lib.extend_attn(bf16_bits(q), kp_in, vp_in, bf16_bits(kc), bf16_bits(vc), 0.1,
                                            n_threads=4)
    units = [5, 17, 40, 95]
    part, part_lse = oracle_lib.extend_attn(bf16_bits(q), kp_in, vp_in, bf16_bits(kc), bf16_bits(vc), 0.1,
                                            units=units)
    for u in units:
        assert np.array_equal(part[u // hq, u % hq], full[u // hq, u % hq])
        assert part_lse[u // hq, u % hq] == full_lse[u // hq, u % hq]
    assert np.isnan(part[0, 0, 0])
