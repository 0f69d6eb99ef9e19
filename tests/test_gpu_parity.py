"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on seeded
inputs small enough for the oracle: several pages, ragged tails, edge cases.

Bars: quantized bytes and the dequantized workspace are bit-exact; attention
outputs pass |gpu - ref| <= 2e-3 + 1e-2 |ref| against the fp64 oracle over the
dequantized cache."""
import math

import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import (assert_close, bf16_bits, gpu_pool_from_kv, oracle_pool_from_kv, run_decode)

pytestmark = pytest.mark.gpu


def _kv(w, dtype=torch.float32):
    return [tuple(x.to(dtype) for x in W.kv(w, b, 0, int(L))) if L > 0 else
            (torch.zeros((0, w.num_kv_heads, 128), dtype=dtype), torch.zeros((0, w.num_kv_heads, 128), dtype=dtype))
            for b, L in enumerate(w.seq_lens)]


def _oracle_attn(w, opool, q, sm_scale=None, g=1.0):
    return oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, w.num_kv_heads,
                              w.sm_scale if sm_scale is None else sm_scale, g=g, n_threads=8)


CASES = [
    # name, Hq, Hkv, lengths, splits
    ("tiny_gqa8_2k", 8, 1, [2048], 0),
    ("ragged_tails", 8, 2, [1, 15, 16, 17, 33, 100], 3),
    ("llama_shape", 64, 8, [300, 1000], 0),
    ("group16", 16, 1, [77], 4),
    ("group1", 4, 4, [50], 2),
    ("group3", 12, 4, [65, 2], 0),
    ("many_splits", 8, 1, [4096], 64),
    ("one_split", 16, 2, [513], 1),
    # the combine spreads more than 64 splits over several waves of a workgroup
    ("splits_200", 8, 1, [4096, 3000, 17], 200),
    ("splits_1100", 8, 2, [20000, 900], 1100),
]


@pytest.mark.parametrize("name,hq,hkv,lens,splits", CASES, ids=[c[0] for c in CASES])
def test_quantize_and_decode_match_oracle(name, hq, hkv, lens, splits):
    w = W.small_workload(100 + len(name), len(lens), hq, hkv, lens, num_splits=splits, name=name)
    print(f"case {name}: Hq={hq} Hkv={hkv} lens={lens} splits={splits}", flush=True)
    kv = _kv(w)
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    gbytes = gpool.data.cpu().numpy()
    assert np.array_equal(gbytes, opool), f"pool bytes differ at {np.flatnonzero(gbytes != opool)[:8]}"
    q = W.query(w)
    out, lse = run_decode(w, gpool, q, num_splits=splits)
    ref, ref_lse = _oracle_attn(w, opool, q)
    err = assert_close(out.cpu().numpy(), ref, what=name)
    assert_close(lse.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4, what=name + " lse")
    print(f"  max abs err {err:.3e}")


def test_bf16_output_and_bf16_source():
    w = W.small_workload(200, 3, 16, 2, [40, 129, 7], name="bf16")
    kv = _kv(w, torch.bfloat16)
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    q = W.query(w)
    out, _ = run_decode(w, gpool, q, out_dtype=torch.bfloat16)
    ref, _ = _oracle_attn(w, opool, q)
    assert out.dtype == torch.bfloat16
    assert_close(out.float().cpu().numpy(), ref, what="bf16 out")


def _threshold_blocks():
    """Rows of 128 fp32 values whose 16-value blocks sit on every rounding edge:
    amax on each E4M3 midpoint of amax/6 and one ulp either side, and elements on
    each E2M1 midpoint (times the block scale) and one ulp either side."""
    vals = [oracle.e4m3_value(k) for k in range(127)]
    blocks = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for s in range(1, 127):
        D = vals[s]
        amax = np.float32(6 * D)
        elems = []
        for m in mids:
            t = np.float32(m * D)
            elems += [t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf))]
        elems.append(np.float32(0.0))  # 22 elements: two blocks of amax + 11 + 4 negated
        for part in range(2):
            blk = [amax] + elems[part * 11:(part + 1) * 11]
            blk += [-x for x in blk[1:5]]
            blocks.append(np.array(blk[:16], dtype=np.float32))
    for k in range(126):
        t = np.float32(3 * (vals[k] + vals[k + 1]))  # 6 * midpoint, exact
        for a in (t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf))):
            blk = np.full(16, np.float32(0.3) * a, dtype=np.float32)
            blk[3] = -a
            blocks.append(blk)
    # specials: zeros, negative zeros, tiny (scale rounds to 0 or subnormal), saturation
    blocks.append(np.zeros(16, np.float32))
    blocks.append(np.full(16, -0.0, np.float32))
    blocks.append(np.array([1e-5, -2e-5] * 8, np.float32))
    blocks.append(np.linspace(-0.004, 0.003, 16).astype(np.float32))
    blocks.append(np.linspace(-5e4, 7e4, 16).astype(np.float32))
    blocks.append(np.array([3e38, -1.0] * 8, np.float32))
    n = len(blocks)
    pad = (-n) % 8
    blocks += [blocks[i % n] * np.float32(1.5) for i in range(pad)]
    return np.stack(blocks).reshape(-1, 1, 128)


def test_quantize_rounding_edges_bitexact():
    rows = _threshold_blocks()  # [T, 1, 128]
    T = rows.shape[0]
    w = W.small_workload(300, 1, 1, 1, [T], name="edges")
    k = torch.from_numpy(rows)
    v = torch.from_numpy(rows[::-1].copy())
    gpool = gpu_pool_from_kv(w, [(k, v)])
    opool = oracle_pool_from_kv(w, [(k, v)])
    g = gpool.data.cpu().numpy()
    assert np.array_equal(g, opool), f"{int((g != opool).sum())} bytes differ"


def _special_rows(T, seed):
    """[T, 2, 128] fp32 rows: seeded N(0,1) values with blocks that hold NaN (both
    signs), infinities, values whose block scale saturates, blocks whose scale
    rounds to zero, and a NaN among finite values (ignored by amax)."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, 2, 128)).astype(np.float32)
    nan = np.float32(np.nan)
    x[0, 0, 3] = nan
    x[1, 1, 17] = -nan
    x[2, 0, 40] = np.inf
    x[3, 1, 64] = -np.inf
    x[4, 0, 80:96] = np.float32(3e38) * np.sign(x[4, 0, 80:96])
    x[5, 1, 0:16] = np.float32(1e-30) * x[5, 1, 0:16]
    x[6, 0, 96:112] = np.float32(5000.0) * x[6, 0, 96:112]
    x[7, 1, 112:128] = nan
    x[8, 0, 16:32] = -0.0
    for t in range(9, T, 7):  # more of the same further on, in whole pages and tails
        x[t, t % 2, (t * 5) % 128] = nan if t % 3 else -np.inf
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_special_values_bitexact(dtype):
    """NaN, infinities, saturated and zero block scales through the whole-page
    writer (tokens filling pages in order), the per-block writer (a call that
    starts mid-page, and the partial last page) and the four-row V groups: the
    pool bytes equal the oracle's."""
    w = W.small_workload(500, 2, 4, 2, [48, 37], name="specials")
    rows = [torch.from_numpy(_special_rows(int(L), 77 + b)) for b, L in enumerate(w.seq_lens)]
    kv = [(r.to(dtype), r.flip(0).contiguous().to(dtype)) for r in rows]
    pool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda")
    # sequence 0 in one call; sequence 1 as tokens [0, 5) and [5, 37) (not page-aligned)
    for b, cuts in ((0, [(0, 48)]), (1, [(0, 5), (5, 37)])):
        for t0, t1 in cuts:
            k, v = kv[b]
            slots = torch.as_tensor(W.slots(w, b, t0, t1), device="cuda")
            B.nvfp4_kv_quantize(k[t0:t1].cuda().contiguous(), v[t0:t1].cuda().contiguous(), slots, pool)
    torch.cuda.synchronize()
    opool = oracle_pool_from_kv(w, kv)
    gp = pool.data.cpu().numpy()
    assert np.array_equal(gp, opool), f"{int((gp != opool).sum())} bytes differ"


@pytest.mark.parametrize("pattern", ["in_order", "reversed", "gap", "mid_page", "mixed_seqs"])
def test_quantize_slot_patterns_bitexact(pattern):
    """The quantize kernel writes a (page, head) slab whole when one 16-token group
    of the call fills a page in order, and block by block otherwise. Every way a
    group can miss the whole-page case must still give the oracle's bytes:
    tokens in reverse order, a skipped slot (-1) inside a page group, a call that
    starts mid-page, and one call holding tokens of several sequences."""
    w = W.small_workload(700, 3, 8, 2, [64, 40, 23], name="slots")
    kv = _kv(w, torch.bfloat16)
    calls = []  # (k, v, slots) per call
    if pattern == "in_order":
        calls = [(k, v, W.slots(w, b, 0, int(L))) for b, ((k, v), L) in enumerate(zip(kv, w.seq_lens))]
    elif pattern == "reversed":
        for b, ((k, v), L) in enumerate(zip(kv, w.seq_lens)):
            calls.append((k.flip(0), v.flip(0), W.slots(w, b, 0, int(L))[::-1].copy()))
    elif pattern == "gap":
        for b, ((k, v), L) in enumerate(zip(kv, w.seq_lens)):
            sl = W.slots(w, b, 0, int(L)).copy()
            sl[5] = -1  # token 5 of every sequence is not written by this call
            calls.append((k, v, sl))
        # the skipped tokens in a second call (each alone in its V group)
        for b, ((k, v), L) in enumerate(zip(kv, w.seq_lens)):
            calls.append((k[5:6], v[5:6], W.slots(w, b, 5, 6)))
    elif pattern == "mid_page":
        for b, ((k, v), L) in enumerate(zip(kv, w.seq_lens)):
            cut = min(7, int(L))
            calls.append((k[:cut], v[:cut], W.slots(w, b, 0, cut)))
            calls.append((k[cut:], v[cut:], W.slots(w, b, cut, int(L))))
    else:  # mixed_seqs: all sequences in one call, so groups straddle sequences
        calls = [(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]),
                  np.concatenate([W.slots(w, b, 0, int(L)) for b, L in enumerate(w.seq_lens)]))]
    pool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda")
    opool = np.zeros(oracle.pool_bytes(w.num_pages, w.num_kv_heads), dtype=np.uint8)
    for k, v, sl in calls:
        B.nvfp4_kv_quantize(k.cuda().contiguous(), v.cuda().contiguous(),
                            torch.as_tensor(np.ascontiguousarray(sl), device="cuda"), pool)
        oracle.quantize_to_pool(bf16_bits(k), bf16_bits(v), np.ascontiguousarray(sl), w.num_pages, pool=opool)
    torch.cuda.synchronize()
    gp = pool.data.cpu().numpy()
    assert np.array_equal(gp, opool), f"{pattern}: {int((gp != opool).sum())} bytes differ"


@pytest.mark.parametrize("g", [0.5, 4.0])
def test_power_of_two_global_scale(g):
    w = W.small_workload(400, 2, 8, 1, [70, 33], name="gscale")
    kv = [(k * g, v * g) for k, v in _kv(w)]
    gpool = gpu_pool_from_kv(w, kv, g=g)
    opool = oracle_pool_from_kv(w, kv, g=g)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    q = W.query(w)
    out, lse = run_decode(w, gpool, q, sm_scale=w.sm_scale / g)
    ref, _ = _oracle_attn(w, opool, q, sm_scale=w.sm_scale / g, g=g)
    assert_close(out.cpu().numpy(), ref, atol=2e-3 * g, what=f"g={g}")
    # the same bytes under g = 1 give exactly 1/g of the output (logits kept equal)
    pool1 = B.Pool(w.num_pages, 1, global_scale=1.0, data=gpool.data)
    out1, _ = run_decode(w, pool1, q)
    assert torch.equal(out, out1 * g)


def test_dequant_workspace_bitexact():
    lens = [37, 16, 200]
    w = W.small_workload(500, 3, 8, 2, lens, name="dequant")
    kv = _kv(w)
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    ko, vo = oracle.dequant_workspace(opool, 2, w.page_table, w.seq_lens)
    rows = int(sum(lens))
    pt = torch.as_tensor(w.page_table, device="cuda")
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    ro = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64), device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        k_out = torch.full((rows, 2, 128), float("nan"), dtype=dt, device="cuda")
        v_out = torch.full_like(k_out, float("nan"))
        B.nvfp4_kv_dequant_workspace(gpool, pt, sl, ro, max(lens), k_out, v_out)
        torch.cuda.synchronize()
        for got, ref in ((k_out, ko), (v_out, vo)):
            want = torch.from_numpy(ref).to(dt)  # exact: at most 6 significant bits
            assert torch.equal(want.double(), torch.from_numpy(ref))
            assert torch.equal(got.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               want.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    # FP8 E4M3 workspace: each value's code is the oracle's rounding of its exact
    # value (nearest, ties to even, saturating at 448); scales of 2^-2 .. 2^7
    # times large codes exceed 448 in places, so saturation is exercised too
    big = [(k * 64.0, v * 64.0) for k, v in kv]
    gbig = gpu_pool_from_kv(w, big)
    obig = oracle_pool_from_kv(w, big)
    assert np.array_equal(gbig.data.cpu().numpy(), obig)
    # values scaled by 2^-8: block scales near 2^-9, so dequantized values land on
    # E4M3 subnormals (multiples of 2^-9), with ties between them
    tiny = [(k * 2.0 ** -8, v * 2.0 ** -8) for k, v in kv]
    gtiny = gpu_pool_from_kv(w, tiny)
    otiny = oracle_pool_from_kv(w, tiny)
    assert np.array_equal(gtiny.data.cpu().numpy(), otiny)
    for pool_g, pool_o in ((gpool, opool), (gbig, obig), (gtiny, otiny)):
        kr, vr = oracle.dequant_workspace(pool_o, 2, w.page_table, w.seq_lens)
        k8 = torch.full((rows, 2, 128), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        v8 = torch.full_like(k8.view(torch.uint8), 0x7F).view(torch.float8_e4m3fn)
        B.nvfp4_kv_dequant_workspace(pool_g, pt, sl, ro, max(lens), k8, v8)
        torch.cuda.synchronize()
        for got, ref in ((k8, kr), (v8, vr)):
            want = oracle.e4m3_codes_of(ref)
            gotb = got.view(torch.uint8).cpu().numpy()
            assert np.array_equal(gotb, want), f"{int((gotb != want).sum())} FP8 codes differ"
        if pool_g is gbig:
            assert np.abs(kr).max() > 448  # saturation was exercised
        if pool_g is gtiny:  # subnormal E4M3 results, some of them ties, were exercised
            a = np.abs(kr[kr != 0])
            assert (a < 2.0 ** -6).mean() > 0.2
            assert np.any((a * 2.0 ** 9) % 1 == 0.5)


def test_split_count_and_page_permutation_invariance_and_reproducibility():
    lens = [700, 333]
    w1 = W.small_workload(600, 2, 16, 2, lens, name="inv1")
    w2 = W.small_workload(601, 2, 16, 2, lens, name="inv2")
    kv = _kv(w1)
    p1 = gpu_pool_from_kv(w1, kv)
    p2 = gpu_pool_from_kv(w2, kv)
    q = W.query(w1)
    a, la = run_decode(w1, p1, q, num_splits=3)
    b, lb = run_decode(w2, p2, q, num_splits=3)
    assert torch.equal(a, b) and torch.equal(la, lb)  # physical placement does not matter
    for _ in range(3):
        c, lc = run_decode(w1, p1, q, num_splits=3)
        assert torch.equal(a, c) and torch.equal(la, lc)  # bit-reproducible
    for s in (1, 2, 7, 11, 0):
        d, ld = run_decode(w1, p1, q, num_splits=s)
        # splits round P to f16 against different running maxima: |dP|/P <= 2^-11
        assert torch.allclose(a, d, atol=1e-3, rtol=1e-3), s
        assert torch.allclose(la, ld, atol=1e-5, rtol=1e-5), s


def test_empty_and_single_token_sequences():
    lens = [0, 1, 16, 0]
    w = W.small_workload(700, 4, 8, 1, lens, name="empty")
    kv = _kv(w)
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    q = W.query(w)
    out, lse = run_decode(w, gpool, q, num_splits=4)
    o, l = out.cpu(), lse.cpu()
    assert torch.all(o[0] == 0) and torch.all(o[3] == 0)
    assert torch.all(torch.isneginf(l[0])) and torch.all(torch.isneginf(l[3]))
    ref, _ = _oracle_attn(w, opool, q)
    assert_close(o[1:3].numpy(), ref[1:3], what="len 1/16")
    vrow = oracle.dequant_row(opool, w.page_table[1, 0], 0, 0, 1, 1)
    assert np.allclose(o[1].numpy(), np.broadcast_to(vrow, (8, 128)), rtol=1e-6, atol=1e-7)


def test_representable_kv_against_dense_attention():
    """K/V built from representable blocks: the NVFP4 cache holds them exactly, so the
    GPU output must match dense fp64 attention over the original values."""
    rng = np.random.default_rng(5)
    lens = [333, 64]
    w = W.small_workload(800, 2, 16, 2, lens, name="repr")
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    kv = []
    for L in lens:
        pair = []
        for _ in range(2):
            codes = rng.integers(0, 16, size=(L, 2, 8, 16))
            codes[..., 0] = 7
            vals = mags[codes & 7] * np.where(codes & 8, -1, 1)
            sc = np.array([oracle.e4m3_value(int(b)) for b in rng.integers(0x28, 0x48, size=L * 16)]).reshape(L, 2, 8)
            pair.append(torch.from_numpy((vals * sc[..., None]).reshape(L, 2, 128).astype(np.float32)))
        kv.append(tuple(pair))
    gpool = gpu_pool_from_kv(w, kv)
    q = W.query(w)
    out, _ = run_decode(w, gpool, q)
    for b, (k, v) in enumerate(kv):
        qq = q[b].double().unsqueeze(1)
        kk = k.double().permute(1, 0, 2).repeat_interleave(8, 0)
        vv = v.double().permute(1, 0, 2).repeat_interleave(8, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=w.sm_scale).squeeze(1)
        assert_close(out[b].cpu().numpy(), ref.numpy(), what=f"dense seq {b}")


@pytest.mark.parametrize("kscale,qscale", [(3e-3, 1.0), (1.0, 3e3), (1.0, 1e-6), (50.0, 1.0)])
def test_extreme_magnitudes(kscale, qscale):
    """Tiny K/V (subnormal E4M3 scales and f16 subnormals in the dequantized
    values), large or tiny queries (the query rescale), large K/V."""
    lens = [90, 31]
    w = W.small_workload(900, 2, 8, 1, lens, name="mag")
    kv = [(k * kscale, v * kscale) for k, v in _kv(w)]
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    assert np.array_equal(gpool.data.cpu().numpy(), opool)
    q = (W.query(w).float() * qscale).to(torch.bfloat16)
    out, lse = run_decode(w, gpool, q)
    ref, ref_lse = _oracle_attn(w, opool, q)
    assert_close(out.cpu().numpy(), ref, atol=2e-3 * kscale, what=f"k x{kscale} q x{qscale}")
    assert_close(lse.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4, what="lse")


def test_partial_states_cover_every_token_once_and_match_oracle():
    """Phase 1 on its own: each non-empty state s covers the tokens of splits
    s .. t-1 (t = the next non-empty state, or S), as the C header documents, and
    matches the oracle over exactly those tokens; empty states are (-inf, 0); the
    states together give the full call's output. 4 x 8 (sequence, KV head) x 64
    splits are more units than resident workgroups, so runs of several splits
    (merged into one state) occur."""
    lens = [2048, 1500, 2048, 700]
    S = 64
    w = W.small_workload(321, len(lens), 64, 8, lens, name="partial_states")
    kv = _kv(w)
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    q = W.query(w)
    pt = torch.as_tensor(w.page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    Bn, Hq = w.batch, w.num_q_heads
    ws = torch.empty(B.nvfp4_paged_decode_attn_workspace_bytes(Bn, Hq, S), dtype=torch.uint8, device="cuda")
    B.nvfp4_paged_decode_attn_partial(q.cuda(), pt, sl, gpool, w.sm_scale, w.max_seq_len, S, ws)
    torch.cuda.synchronize()
    wsf = ws.view(torch.float32).cpu().numpy()
    n_o = Bn * Hq * S * 128
    O = wsf[:n_o].reshape(Bn, Hq, S, 128).astype(np.float64)
    ML = wsf[n_o:n_o + Bn * Hq * S * 2].reshape(Bn, Hq, S, 2).astype(np.float64)
    M, Z = ML[..., 0], ML[..., 1]
    empty = np.isneginf(M)
    assert np.all(Z[empty] == 0) and np.all(Z[~empty] > 0) and np.all(np.isfinite(M[~empty]))
    # every query head of a KV group shares the decomposition
    grp = Hq // w.num_kv_heads
    for h in range(w.num_kv_heads):
        assert np.array_equal(empty[:, h * grp:(h + 1) * grp], np.repeat(empty[:, h * grp:h * grp + 1], grp, axis=1))
    merged = 0
    rows, seq_lens, owners = [], [], []
    for b, L in enumerate(lens):
        n_b = -(-L // 16)
        P = -(-n_b // S)
        for h in range(w.num_kv_heads):
            live = [s for s in range(S) if not empty[b, h * grp, s]]
            for i, s in enumerate(live):
                t = live[i + 1] if i + 1 < len(live) else S
                merged += t - s > 1 and min(t * P, n_b) > min((s + 1) * P, n_b)
                p0, p1 = min(s * P, n_b), min(t * P, n_b)
                assert p1 > p0, (b, h, s, t)
                row = np.full(w.page_table.shape[1], -1, dtype=np.int32)
                row[:p1 - p0] = w.page_table[b, p0:p1]
                rows.append(row)
                seq_lens.append(min(L, p1 * 16) - p0 * 16)
                owners.append((b, h, s))
            # the live states' ranges tile the sequence: pages before the first
            # live state belong to no state only if they do not exist
            assert not live or min(live[0] * P, n_b) == 0
    assert merged > 0, "no state covered several splits"
    # oracle over each state's tokens: one virtual sequence per (b, h, state)
    vpt = np.stack(rows)
    vlen = np.asarray(seq_lens, dtype=np.int32)
    qv = torch.stack([q[b, h * grp:(h + 1) * grp] for b, h, _ in owners])  # [V, grp, 128]
    ref, ref_lse = _oracle_per_head(w, opool, qv, vpt, vlen, owners)
    for i, (b, h, s) in enumerate(owners):
        heads = slice(h * grp, (h + 1) * grp)
        got = O[b, heads, s] / Z[b, heads, s][:, None]
        assert_close(got, ref[i], what=f"state b={b} h={h} s={s}")
        lse_state = (M[b, heads, s] + np.log2(Z[b, heads, s])) * math.log(2.0)
        assert_close(lse_state, ref_lse[i], atol=1e-3, rtol=1e-4, what=f"state lse b={b} h={h} s={s}")
    # the combine of these states is the full call's output
    out = torch.empty((Bn, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((Bn, Hq), dtype=torch.float32, device="cuda")
    B.nvfp4_decode_combine(ws, Bn, Hq, S, out, lse=lse)
    full_out, full_lse = run_decode(w, gpool, q, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(out, full_out) and torch.equal(lse, full_lse)


def _oracle_per_head(w, opool, qv, vpt, vlen, owners):
    """Oracle attention of each virtual sequence for the query heads of its own KV
    head: run with the workload's KV-head count, the group's queries placed at
    their head and zeros elsewhere, then keep the owner head's rows."""
    grp = w.num_q_heads // w.num_kv_heads
    V = len(owners)
    qfull = torch.zeros((V, w.num_q_heads, 128), dtype=torch.bfloat16)
    units = []
    for i, (_, h, _) in enumerate(owners):
        qfull[i, h * grp:(h + 1) * grp] = qv[i]
        units += [i * w.num_q_heads + h * grp + g for g in range(grp)]
    out, lse = oracle.decode_attn(bf16_bits(qfull), vpt, vlen, opool, w.num_kv_heads, w.sm_scale, units=units,
                                  n_threads=8)
    ref = np.stack([out[i, h * grp:(h + 1) * grp] for i, (_, h, _) in enumerate(owners)])
    ref_lse = np.stack([lse[i, h * grp:(h + 1) * grp] for i, (_, h, _) in enumerate(owners)])
    return ref, ref_lse


def test_quantize_write_orders_give_the_oracle_bytes():
    """A V code byte holds two rows of a page: whole four-row groups written by one
    call take the grouped path, single tokens and broken groups the per-nibble
    atomic path. Any mix of them, in any order, over stale bytes, must leave the
    oracle's bytes (the oracle writes everything in one call)."""
    lens = [70, 45, 16]
    w = W.small_workload(500, len(lens), 8, 2, lens, name="write_orders")
    kv = _kv(w)
    opool = oracle_pool_from_kv(w, kv)
    rng = np.random.default_rng(7)
    gpool = B.Pool(w.num_pages, w.num_kv_heads, device="cuda",
                   data=torch.full((opool.size,), 0xA5, dtype=torch.uint8, device="cuda"))
    for b, (k, v) in enumerate(kv):
        L = k.shape[0]
        slots = W.slots(w, b, 0, L)
        t = 0
        calls = []
        while t < L:  # cut the sequence into runs of 1..9 tokens
            n = int(rng.integers(1, 10))
            calls.append(np.arange(t, min(L, t + n)))
            t += n
        rng.shuffle(calls)
        for idx in calls:
            if rng.random() < 0.3:
                idx = idx[::-1].copy()  # reversed: groups are not consecutive in the call
            ti = torch.as_tensor(idx)
            kk = k[ti].cuda().contiguous()
            vv = v[ti].cuda().contiguous()
            B.nvfp4_kv_quantize(kk, vv, torch.as_tensor(slots[idx], device="cuda"), gpool)
    # one call with a skipped token (slot -1) in the middle of a group
    k0, v0 = kv[2]
    sl = W.slots(w, 2, 0, 16).copy()
    sl[5] = -1
    B.nvfp4_kv_quantize(k0.cuda().contiguous(), v0.cuda().contiguous(), torch.as_tensor(sl, device="cuda"), gpool)
    B.nvfp4_kv_quantize(k0[5:6].cuda().contiguous(), v0[5:6].cuda().contiguous(),
                        torch.as_tensor(W.slots(w, 2, 5, 6), device="cuda"), gpool)
    torch.cuda.synchronize()
    g = gpool.data.cpu().numpy()
    # compare the bytes every written token owns: whole slabs of fully written
    # pages, and for partly written pages the dequantized tokens
    ko, vo = oracle.dequant_workspace(g, w.num_kv_heads, w.page_table, w.seq_lens)
    kr, vr = oracle.dequant_workspace(opool, w.num_kv_heads, w.page_table, w.seq_lens)
    assert np.array_equal(ko, kr) and np.array_equal(vo, vr)
    full_pages = [int(p) for b, L in enumerate(lens) for p in w.page_table[b, :L // 16]]
    for p in full_pages:
        o = oracle.slab_offset(p, 0, 0, w.num_kv_heads)
        span = w.num_kv_heads * 2 * 1152
        assert np.array_equal(g[o:o + span], opool[o:o + span]), f"page {p}"


@pytest.mark.parametrize("fp8", [False, True], ids=["nvfp4", "fp8"])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_wide_page_table_parity(fp8, splits):
    """A page table far wider than the sequences (max_seq_len 32768 for sequences
    of 0 to 3000 tokens, so the default split count gives splits of one page and
    many empty ones), checked against the oracle on every output; a second call
    gives bit-identical results."""
    lens = [3000, 1, 0, 517, 1600, 33]
    hq, hkv = 64, 8
    w = W.small_workload(611, len(lens), hq, hkv, lens, num_splits=splits, name="wide_table")
    stride = 2048
    pt_wide = np.full((w.batch, stride), 0, dtype=np.int32)
    pt_wide[:, :w.page_table.shape[1]] = w.page_table
    max_len = stride * 16
    kv = _kv(w)
    q = W.query(w)
    if fp8:
        gpool = B.Fp8Pool(w.num_pages, hkv, device="cuda")
        opool = np.zeros(oracle.fp8_pool_bytes(w.num_pages, hkv), dtype=np.uint8)
        for b, (k, v) in enumerate(kv):
            if k.shape[0]:
                sl_b = W.slots(w, b, 0, k.shape[0])
                B.fp8_kv_quantize(k.cuda().contiguous(), v.cuda().contiguous(), torch.as_tensor(sl_b, device="cuda"),
                                  gpool)
                oracle.fp8_quantize_to_pool(k.numpy(), v.numpy(), sl_b, w.num_pages, pool=opool)
        torch.cuda.synchronize()
        fn, default = B.fp8_paged_decode_attn, B.fp8_paged_decode_attn_default_splits
        ref, ref_lse = oracle.fp8_decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale,
                                              n_threads=8)
    else:
        gpool = gpu_pool_from_kv(w, kv)
        opool = oracle_pool_from_kv(w, kv)
        fn, default = B.nvfp4_paged_decode_attn, B.nvfp4_paged_decode_attn_default_splits
        ref, ref_lse = oracle.decode_attn(bf16_bits(q), w.page_table, w.seq_lens, opool, hkv, w.sm_scale, n_threads=8)
    S = splits or default(w.batch, hkv, max_len)
    ws = torch.empty(B.nvfp4_paged_decode_attn_workspace_bytes(w.batch, hq, S), dtype=torch.uint8, device="cuda")
    pt = torch.as_tensor(pt_wide, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    results = []
    for _ in range(2):
        lse = torch.empty((w.batch, hq), dtype=torch.float32, device="cuda")
        out = fn(q.cuda().contiguous(), pt, sl, gpool, w.sm_scale, max_len, num_splits=S, workspace=ws,
                 out_dtype=torch.float32, lse=lse)
        torch.cuda.synchronize()
        results.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(results[0][0], results[1][0]) and np.array_equal(results[0][1], results[1][1])
    out, lse = results[0]
    live = np.asarray(w.seq_lens) > 0
    assert_close(out[live], ref[live], what=f"wide page table splits={S}")
    assert_close(lse[live], ref_lse[live], atol=1e-3, rtol=1e-4, what="lse")
    assert np.all(out[~live] == 0) and np.all(np.isneginf(lse[~live]))
