"""Pins of the oracle's FP8 baseline: E4M3 codes of x / s against torch's
float8_e4m3fn cast, saturation and signed zeros in closed form, the pool layout
as a bijection, exact round trips, and decode attention over an FP8 pool against
torch's fp64 scaled_dot_product_attention on E4M3-representable K/V."""
import numpy as np
import pytest
import torch

from bit_paged_kv_nvfp4_amd import workload as W
from tests.test_oracle_attention import bf16_bits, sdpa_ref

SCALES = [1.0, 0.5, 4.0]


def e4m3_all_finite():
    b = np.array([x for x in range(256) if (x & 0x7F) != 0x7F], dtype=np.uint8)
    return torch.tensor(b).view(torch.float8_e4m3fn).float().numpy()


def test_fp8_layout_is_a_bijection(oracle_lib):
    for kind in (0, 1):
        offs = {oracle_lib.fp8_byte_offset(kind, r, d) for r in range(16) for d in range(128)}
        assert offs == set(range(2048))
    # K rows are token-major; a V chunk (32 B) holds channels 8n..8n+7 of rows
    # 4g..4g+3, channel-major (4 rows of one channel in one 32-bit word)
    assert [oracle_lib.fp8_byte_offset(0, 3, d) for d in range(128)] == list(range(384, 512))
    for g in range(4):
        for n in range(16):
            c = 16 * g + n
            for q in range(8):
                word = [oracle_lib.fp8_byte_offset(1, 4 * g + i, 8 * n + q) for i in range(4)]
                assert word == list(range(32 * c + 4 * q, 32 * c + 4 * q + 4))
    assert oracle_lib.fp8_slab_offset(3, 1, 1, 8) == ((3 * 8 + 1) * 2 + 1) * 2048
    assert oracle_lib.fp8_pool_bytes(10, 8) == 10 * 8 * 2 * 2048


@pytest.mark.parametrize("s", SCALES)
def test_fp8_codes_vs_library_cast(oracle_lib, s):
    rng = np.random.default_rng(51)
    vals = e4m3_all_finite().astype(np.float64)
    mags = np.unique(np.abs(vals))
    mids = (mags[:-1] + mags[1:]) / 2  # ties, and one float32 ulp to each side
    pts = np.concatenate([vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                          np.nextafter(mids.astype(np.float32), np.float32(1e9)), rng.uniform(-448, 448, 3000)])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    x = (pts * np.float32(s)).astype(np.float32)  # x / s == pts exactly (power-of-two s)
    ref = torch.tensor(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_lib.fp8_code(float(v), s) for v in x], dtype=np.uint8)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_fp8_codes_saturate_and_keep_sign(oracle_lib):
    assert oracle_lib.fp8_code(448.0) == 0x7E and oracle_lib.fp8_code(-1e6) == 0xFE
    assert oracle_lib.fp8_code(500.0, 0.5) == 0x7E  # 1000 > 448
    assert oracle_lib.fp8_code(1000.0, 4.0) == 0x78  # 250 lies between 240 (0x77) and 256 (0x78): 256
    assert oracle_lib.fp8_code(0.0) == 0x00 and oracle_lib.fp8_code(-0.0) == 0x80
    assert oracle_lib.fp8_code(2.0 ** -10) == 0x00  # half the smallest subnormal: tie to even (0)
    assert oracle_lib.fp8_code(3 * 2.0 ** -10) == 0x02  # 1.5 subnormal steps: tie to even (2)


def _fp8_kv(rng, T, hkv, scale):
    """float32 [T, hkv, 128] of E4M3 values times scale, with 448 present."""
    vals = e4m3_all_finite()
    x = rng.choice(vals[np.abs(vals) <= 64], size=(T, hkv, 128)).astype(np.float32)
    x[0, 0, 0] = 448.0
    return (x * np.float32(scale)).astype(np.float32)


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.5, 2.0)])
def test_fp8_round_trip_and_attention_vs_library_sdpa(oracle_lib, ks, vs):
    rng = np.random.default_rng(52)
    lens = [37, 16, 1]
    hq, hkv = 8, 2
    w = W.small_workload(53, len(lens), hq, hkv, lens)
    kl = [_fp8_kv(rng, L, hkv, ks) for L in lens]
    vl = [_fp8_kv(rng, L, hkv, vs) for L in lens]
    pool = np.zeros(oracle_lib.fp8_pool_bytes(w.num_pages, hkv), dtype=np.uint8)
    for b, L in enumerate(lens):
        oracle_lib.fp8_quantize_to_pool(kl[b], vl[b], W.slots(w, b, 0, L), w.num_pages, ks, vs, pool=pool)
    for b, L in enumerate(lens):
        for t in range(L):
            page, row = w.page_table[b, t // 16], t % 16
            for h in range(hkv):
                assert np.array_equal(oracle_lib.fp8_dequant_row(pool, page, row, h, 0, hkv, ks), kl[b][t, h])
                assert np.array_equal(oracle_lib.fp8_dequant_row(pool, page, row, h, 1, hkv, vs), vl[b][t, h])
    q = W.query(w)
    sm = 128 ** -0.5 / 16  # keep logits moderate for K values up to 448
    out, lse = oracle_lib.fp8_decode_attn(bf16_bits(q), w.page_table, w.seq_lens, pool, hkv, sm, ks, vs)
    ref, ref_lse = sdpa_ref(q, kl, vl, hq, hkv, sm)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
