"""GPU parity at global scales that are not powers of two (the per-tensor FP32
scale of page "NVFP4-KV-Cache auf der NVIDIA RTX PRO 6000 Blackwell Server
Edition", section "Bytes pro Token"), through the C ABI, against the oracle.

Bars: pool bytes bit-exact (every scale and code decision is the one on the
exact quotient); a dense workspace holds the nearest value of its dtype to the
exact E2M1 * E4M3 * g (bit-exact against the oracle's one rounding); attention
within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the fp64 oracle."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import assert_close, bf16_bits, gpu_pool_from_kv, oracle_pool_from_kv, run_decode

pytestmark = pytest.mark.gpu

G_VALUES = [float(np.float32(0.3)), float(np.float32(1 / 2688)), 7.5]
MIDS = [Fraction(m) for m in ("1/4", "3/4", "5/4", "7/4", "5/2", "7/2", "5")]


def _e4m3(b):
    return Fraction(oracle.e4m3_value(b))


def _near(q: Fraction):
    t = np.float32(float(q))
    return [t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf))]


def _edge_rows(g, seed):
    """float32 rows [T, 1, 128] of 16-value blocks on the decision edges for g:
    (a) the block maximum on every E4M3 midpoint times 6 g (+-1 ulp), (b) for
    several scales s, a block whose other values sit on every E2M1 midpoint times
    E4M3(s) g (+-1 ulp), both signs; then seeded N(0, 1) rows times g."""
    rng = np.random.default_rng(seed)
    G = Fraction(g)
    blocks = []
    for k in range(126):
        mid = (_e4m3(k) + _e4m3(k + 1)) / 2
        for a in _near(mid * 6 * G):
            x = (rng.uniform(-1, 1, 16) * float(a)).astype(np.float32)
            x[int(rng.integers(0, 16))] = a * np.float32(1 if rng.random() < 0.5 else -1)
            blocks.append(x)
    for s in (3, 9, 20, 45, 60, 77, 90, 110, 126):
        D = _e4m3(s) * G
        vals = [v for m in MIDS for v in _near(m * D)]  # 21 values
        for part in (vals[:15], vals[6:]):
            x = np.zeros(16, np.float32)
            x[0] = np.float32(float(6 * D))
            x[1:] = [v if i % 2 else -v for i, v in enumerate(part)]
            blocks.append(x)
    while len(blocks) % 8:
        blocks.append(blocks[-1] * np.float32(0.75))
    rows = np.stack(blocks).reshape(-1, 1, 128)
    noise = (rng.standard_normal((24, 1, 128)) * g).astype(np.float32)
    return np.concatenate([rows, noise])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("g", G_VALUES)
def test_quantize_any_global_scale_bitexact(g, dtype):
    """Every decision edge of g, through the whole-page writer (a sequence in one
    call), the per-block writer (a call that starts mid-page) and single tokens
    (the V nibbles by atomics)."""
    print(f"quantize g={g} {dtype}", flush=True)
    rows = torch.from_numpy(_edge_rows(g, int(g * 1e6) % 1000))
    T = rows.shape[0]
    w = W.small_workload(810, 3, 1, 1, [T, T, T], name="anyg")
    kv = [(rows.to(dtype), rows.flip(0).contiguous().to(dtype))] * 3
    pool = B.Pool(w.num_pages, 1, device="cuda", global_scale=g)
    cuts = {0: [(0, T)], 1: [(0, 7), (7, T)], 2: [(t, t + 1) for t in range(0, T, 37)]}
    opool = np.zeros(oracle.pool_bytes(w.num_pages, 1), dtype=np.uint8)
    for b, cs in cuts.items():
        k, v = kv[b]
        for t0, t1 in cs:
            sl = W.slots(w, b, t0, t1)
            B.nvfp4_kv_quantize(k[t0:t1].cuda().contiguous(), v[t0:t1].cuda().contiguous(),
                                torch.as_tensor(sl, device="cuda"), pool)
            kk, vv = (bf16_bits(k[t0:t1]), bf16_bits(v[t0:t1])) if dtype == torch.bfloat16 else \
                (k[t0:t1].numpy(), v[t0:t1].numpy())
            oracle.quantize_to_pool(kk, vv, sl, w.num_pages, g=g, pool=opool)
    torch.cuda.synchronize()
    gp = pool.data.cpu().numpy()
    assert np.array_equal(gp, opool), f"g={g}: {int((gp != opool).sum())} bytes differ"


@pytest.mark.parametrize("g", [float(np.float32(0.3)), 7.5])
def test_decode_and_fused_step_any_global_scale(g):
    lens = [300, 47, 1000]
    w = W.small_workload(820, 3, 16, 2, lens, name="anyg_decode")
    kv = [(k * g, v * g) for k, v in (W.kv(w, b, 0, L) for b, L in enumerate(lens))]
    gpool = gpu_pool_from_kv(w, kv, g=g)
    opool = oracle_pool_from_kv(w, kv, g=g)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    q = W.query(w)
    sm = w.sm_scale / g  # logits of the original scale
    out, lse = run_decode(w, gpool, q, sm_scale=sm)
    ref, ref_lse = oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, 2, sm, g=g, n_threads=8)
    assert_close(out.cpu().numpy(), ref, atol=2e-3 * g, what=f"decode g={g}")
    assert_close(lse.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4, what="lse")
    # the fused step: the newest token of each sequence written by the split launch
    pool2 = B.Pool(w.num_pages, 2, device="cuda", global_scale=g)
    for b, (k, v) in enumerate(kv):
        L = lens[b]
        B.nvfp4_kv_quantize(k[:L - 1].cuda(), v[:L - 1].cuda(), torch.as_tensor(W.slots(w, b, 0, L - 1),
                                                                                 device="cuda"), pool2)
    kn = torch.stack([k[-1] for k, _ in kv]).cuda()
    vn = torch.stack([v[-1] for _, v in kv]).cuda()
    out2 = B.nvfp4_paged_decode_attn_append(q.cuda(), kn, vn, torch.as_tensor(w.page_table, device="cuda"),
                                            torch.as_tensor(w.seq_lens, device="cuda"), pool2, sm, max(lens),
                                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(pool2.data.cpu().numpy(), opool)
    assert torch.equal(out2, out)


@pytest.mark.parametrize("g", [float(np.float32(0.3)), float(np.float32(1 / 2688)), 7.5])
def test_dequant_workspace_any_global_scale_bitexact(g):
    """f32: the binary32 rounding of the exact value; bf16 and FP8 E4M3: the
    oracle's nearest-even rounding of the exact value (one rounding)."""
    lens = [37, 16, 200]
    w = W.small_workload(830, 3, 8, 2, lens, name="anyg_dequant")
    kv = [(k * g * 40, v * g * 40) for k, v in (W.kv(w, b, 0, L) for b, L in enumerate(lens))]
    gpool = gpu_pool_from_kv(w, kv, g=g)
    opool = oracle_pool_from_kv(w, kv, g=g)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    ko, vo = oracle.dequant_workspace(opool, 2, w.page_table, w.seq_lens, g=g)
    rows = int(sum(lens))
    pt = torch.as_tensor(w.page_table, device="cuda")
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    ro = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64), device="cuda")
    inexact = 0
    for dt in (torch.float32, torch.bfloat16, torch.float8_e4m3fn):
        k_out = torch.zeros((rows, 2, 128), dtype=dt, device="cuda")
        v_out = torch.zeros_like(k_out)
        B.nvfp4_kv_dequant_workspace(gpool, pt, sl, ro, max(lens), k_out, v_out)
        torch.cuda.synchronize()
        for got, ref in ((k_out, ko), (v_out, vo)):
            if dt == torch.float32:
                want = ref.astype(np.float32).view(np.uint32)
                gotb = got.cpu().numpy().view(np.uint32)
                inexact += int((ref.astype(np.float32).astype(np.float64) != ref).sum())
            elif dt == torch.bfloat16:
                want = oracle.bf16_bits_of(ref)
                gotb = bf16_bits(got)
            else:
                want = oracle.e4m3_codes_of(ref)
                gotb = got.view(torch.uint8).cpu().numpy()
            assert np.array_equal(gotb, want), f"g={g} {dt}: {int((gotb != want).sum())} values differ"
    if g != 7.5:  # 7.5 = 1111b x 2^-1: products of at most 10 bits stay exact in binary32
        assert inexact > 0  # the exact products needed rounding to binary32


def test_extend_fused_chunk_write_any_global_scale():
    g = float(np.float32(0.3))
    P, C, hq, hkv = 50, 70, 16, 2
    q, kp, vp, kc, vc = W.extend_inputs(840, P, C, hq, hkv)
    kc, vc = (kc.float() * g).to(torch.bfloat16), (vc.float() * g).to(torch.bfloat16)
    w = W.small_workload(841, 1, hq, hkv, [P + C])
    slots = W.slots(w, 0, P, P + C)
    gpool = B.Pool(w.num_pages, hkv, device="cuda", global_scale=g)
    B.nvfp4_extend_attn(q.cuda(), kp.cuda(), vp.cuda(), kc.cuda(), vc.cuda(), 128 ** -0.5, chunk_pool=gpool,
                        chunk_slots=torch.as_tensor(slots, device="cuda"))
    torch.cuda.synchronize()
    opool = np.zeros(oracle.pool_bytes(w.num_pages, hkv), dtype=np.uint8)
    oracle.quantize_to_pool(bf16_bits(kc), bf16_bits(vc), slots, w.num_pages, g=g, pool=opool)
    gp = gpool.data.cpu().numpy()
    assert np.array_equal(gp, opool), f"{int((gp != opool).sum())} bytes differ"


def test_tight_calibration_end_to_end():
    """The tight binary32 g of K/V of magnitude ~1e5: pool bytes at g equal the
    oracle's, the bf16 workspace is the oracle's rounding, and decode and extend
    attention (with v_bound = 2688 g) are within the bars."""
    lens = [70, 133]
    w = W.small_workload(850, 2, 16, 2, lens, name="tight")
    kv = [(k * 3.7e4, v * 3.3e4) for k, v in (W.kv(w, b, 0, L) for b, L in enumerate(lens))]
    am = max(float(B.nvfp4_kv_amax(k.cuda(), v.cuda()).max()) for k, v in kv)
    g = B.nvfp4kv_global_scale_tight_for_amax(am)
    assert g == oracle.global_scale_tight_for_amax(am) and g > 16
    gpool = gpu_pool_from_kv(w, kv, g=g)
    opool = oracle_pool_from_kv(w, kv, g=g)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    q = W.query(w)
    sm = w.sm_scale / 3.7e4
    out, _ = run_decode(w, gpool, q, sm_scale=sm)
    ref, _ = oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, 2, sm, g=g, n_threads=8)
    assert_close(out.cpu().numpy() / 3.3e4, ref / 3.3e4, what="decode at the tight g")
    # extend over the bf16 workspace of sequence 1 (values up to 2688 g > 65504)
    P = lens[1]
    ko, vo = oracle.dequant_workspace(opool, 2, w.page_table[1:], w.seq_lens[1:], g=g)
    assert np.abs(vo).max() > 65504
    k_ws = torch.zeros((P, 2, 128), dtype=torch.bfloat16, device="cuda")
    v_ws = torch.zeros_like(k_ws)
    B.nvfp4_kv_dequant_workspace(gpool, torch.as_tensor(w.page_table[1:2], device="cuda").contiguous(),
                                 torch.as_tensor(w.seq_lens[1:2], device="cuda"),
                                 torch.zeros(1, dtype=torch.int64, device="cuda"), P, k_ws, v_ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(v_ws), oracle.bf16_bits_of(vo))
    C = 20
    qc, _, _, kc, vc = W.extend_inputs(851, 0, C, 16, 2)
    kc, vc = (kc.float() * 3.7e4).to(torch.bfloat16), (vc.float() * 3.3e4).to(torch.bfloat16)
    lse = torch.empty((C, 16), dtype=torch.float32, device="cuda")
    out = B.nvfp4_extend_attn(qc.cuda(), k_ws, v_ws, kc.cuda(), vc.cuda(), sm, lse=lse, v_bound=2688.0 * g)
    torch.cuda.synchronize()
    oref, olse = oracle.extend_attn(bf16_bits(qc), bf16_bits(k_ws), bf16_bits(v_ws), bf16_bits(kc), bf16_bits(vc),
                                    sm, n_threads=8)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got / 3.3e4, oref / 3.3e4, what="extend with v_bound")
    assert_close(lse.cpu().numpy(), olse, atol=1e-3, rtol=1e-4, what="extend lse")


@pytest.mark.parametrize("scale", [1.0, 2.0 ** 20])
def test_extend_v_bound_scaling(scale):
    """V beyond the f16 range (x 2^20) attends correctly with v_bound; a bound of
    the same data at scale 1 leaves the result bit-identical to v_bound = 0."""
    P, C, hq, hkv = 100, 37, 8, 1
    q, kp, vp, kc, vc = W.extend_inputs(860, P, C, hq, hkv)
    vp, vc = (vp.float() * scale).to(torch.bfloat16), (vc.float() * scale).to(torch.bfloat16)
    vb = float(max(vp.float().abs().max(), vc.float().abs().max()))
    sm = 128 ** -0.5
    out = B.nvfp4_extend_attn(q.cuda(), kp.cuda(), vp.cuda(), kc.cuda(), vc.cuda(), sm, v_bound=vb)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref, _ = oracle.extend_attn(bf16_bits(q), bf16_bits(kp), bf16_bits(vp), bf16_bits(kc), bf16_bits(vc), sm,
                                n_threads=8)
    assert_close(got / scale, ref / scale, what=f"v_bound scale {scale}")
    if scale == 1.0:
        out0 = B.nvfp4_extend_attn(q.cuda(), kp.cuda(), vp.cuda(), kc.cuda(), vc.cuda(), sm)
        torch.cuda.synchronize()
        assert torch.equal(out0, out)
