"""GPU parity of the extend attention (nvfp4_extend_attn, through the C ABI)
against the oracle's fp64 extend attention on the same seeded inputs.

Bar: |gpu - ref| <= 2e-3 + 1e-2 |ref| for the bf16 output; lse within 1e-3 +
1e-4 |ref|. Inputs: a bf16 or FP8 E4M3 prefix workspace and a bf16 chunk, drawn
by the workload module; the pipeline case feeds each side its own quantize and
dequant of the same K/V."""
import numpy as np
import pytest
import torch

import oracle
from bit_paged_kv_nvfp4_amd import binding as B
from bit_paged_kv_nvfp4_amd import workload as W
from tests.gpu_common import assert_close, bf16_bits, gpu_pool_from_kv, oracle_pool_from_kv

pytestmark = pytest.mark.gpu


def _ws_np(t):
    """A workspace tensor as the oracle's input: bf16 bits or FP8 bytes."""
    t = t.cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.view(torch.uint8).numpy()


def _run(q, kp, vp, kc, vc, sm):
    C, hq, _ = q.shape
    lse = torch.empty((C, hq), dtype=torch.float32, device="cuda")
    out = B.nvfp4_extend_attn(q.cuda(), kp.cuda(), vp.cuda(), kc.cuda(), vc.cuda(), sm, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def _oracle(q, kp, vp, kc, vc, sm, units=None):
    return oracle.extend_attn(bf16_bits(q), _ws_np(kp), _ws_np(vp), bf16_bits(kc), bf16_bits(vc), sm, units=units,
                              n_threads=8)


CASES = [
    # name, P, C, Hq, Hkv, prefix dtype, sm_scale
    ("ragged_tiles_gqa8", 100, 37, 8, 1, torch.bfloat16, None),
    ("no_prefix", 0, 70, 16, 2, torch.bfloat16, None),
    ("llama_shape_fp8", 200, 130, 64, 8, torch.float8_e4m3fn, None),
    ("group1", 64, 64, 4, 4, torch.bfloat16, None),
    ("group3_dummy_rows", 33, 5, 48, 16, torch.float8_e4m3fn, None),
    ("group16", 17, 40, 32, 2, torch.bfloat16, None),
    ("negative_scale", 90, 21, 8, 2, torch.bfloat16, -0.05),
    ("single_token_chunk", 300, 1, 8, 1, torch.float8_e4m3fn, None),
]


@pytest.mark.parametrize("name,P,C,hq,hkv,dt,sm", CASES, ids=[c[0] for c in CASES])
def test_extend_attention_matches_oracle(name, P, C, hq, hkv, dt, sm):
    print(f"case {name}: P={P} C={C} Hq={hq} Hkv={hkv} {dt}", flush=True)
    q, kp, vp, kc, vc = W.extend_inputs(300 + P + C, P, C, hq, hkv, prefix_dtype=dt)
    sm = 128 ** -0.5 if sm is None else sm
    out, lse = _run(q, kp, vp, kc, vc, sm)
    ref, ref_lse = _oracle(q, kp, vp, kc, vc, sm)
    err = assert_close(out, ref, what=name)
    assert_close(lse, ref_lse, atol=1e-3, rtol=1e-4, what=name + " lse")
    print(f"  max abs err {err:.3e}")


def test_extend_pipeline_quantize_dequant_attend():
    """quantize-on-write -> dequant of the prefix into a bf16 and an FP8 workspace
    -> attention, each side on its own: the GPU through the library, the oracle
    through its own pool and workspace."""
    P, C, hq, hkv = 150, 45, 16, 2
    w = W.small_workload(410, 1, hq, hkv, [P])
    k, v = W.kv(w, 0, 0, P)
    gpool = gpu_pool_from_kv(w, [(k, v)])
    opool = oracle_pool_from_kv(w, [(k, v)])
    pt = torch.as_tensor(w.page_table, device="cuda").contiguous()
    sl = torch.as_tensor(w.seq_lens, device="cuda")
    ro = torch.zeros(1, dtype=torch.int64, device="cuda")
    ko, vo = oracle.dequant_workspace(opool, hkv, w.page_table, w.seq_lens)  # exact NVFP4 values, fp64
    q, _, _, kc, vc = W.extend_inputs(411, 0, C, hq, hkv)
    sm = 128 ** -0.5
    for dt in (torch.bfloat16, torch.float8_e4m3fn):
        k_ws = torch.empty((P, hkv, 128), dtype=dt, device="cuda")
        v_ws = torch.empty_like(k_ws)
        B.nvfp4_kv_dequant_workspace(gpool, pt, sl, ro, P, k_ws, v_ws)
        out, lse = _run(q, k_ws, v_ws, kc, vc, sm)
        if dt == torch.bfloat16:  # the values have at most 6 significant bits: exact in bf16
            ok = (ko.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            ov = (vo.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        else:
            ok, ov = oracle.e4m3_codes_of(ko), oracle.e4m3_codes_of(vo)
        ref, ref_lse = oracle.extend_attn(bf16_bits(q), ok, ov, bf16_bits(kc), bf16_bits(vc), sm, n_threads=8)
        assert_close(out, ref, what=f"pipeline {dt}")
        assert_close(lse, ref_lse, atol=1e-3, rtol=1e-4, what=f"pipeline {dt} lse")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float8_e4m3fn])
def test_extend_full_size_sampled_rows(dt):
    """The extend request's full shape (163840-token prefix, 8192-token chunk, 64
    query / 8 KV heads) in the launch configuration bench.py times; the oracle
    checks sampled (token, head) rows: first and last tokens, token-block edges."""
    w = W.config(5)
    P, C, hq, hkv = w.extend_prefix, w.extend_chunk, w.num_q_heads, w.num_kv_heads
    print(f"full size P={P} C={C} {dt}", flush=True)
    q, kp, vp, kc, vc = W.extend_inputs(w.seed, P, C, hq, hkv, prefix_dtype=dt, device="cuda")
    out, lse = _run(q, kp, vp, kc, vc, w.sm_scale)
    tokens = [0, 1, 15, 16, 17, 4095, 4096, 8190, 8191]
    heads = [0, 7, 8, 37, 63]
    units = [t * hq + h for t in tokens for h in heads]
    ref, ref_lse = _oracle(q.cpu(), kp.cpu(), vp.cpu(), kc.cpu(), vc.cpu(), w.sm_scale, units=units)
    ti = np.array([u // hq for u in units])
    hi = np.array([u % hq for u in units])
    err = assert_close(out[ti, hi], ref[ti, hi], what="sampled rows (unit order as listed)")
    assert_close(lse[ti, hi], ref_lse[ti, hi], atol=1e-3, rtol=1e-4, what="sampled lse")
    print(f"  max abs err {err:.3e} over {len(units)} rows")


@pytest.mark.parametrize("P,C,hq,hkv", [(50, 70, 16, 2), (64, 33, 8, 1)])
def test_extend_fused_chunk_write_bytes_and_output(P, C, hq, hkv):
    """With a pool, the extend launch also quantize-writes the chunk: its bytes
    equal the oracle's quantize of the same chunk (over the same stale bytes;
    P = 50 leaves the first four-row V group incomplete, so both the grouped and
    the single-row V writes run), and the attention output is the same as
    without the write."""
    print(f"fused write P={P} C={C} Hq={hq} Hkv={hkv}", flush=True)
    q, kp, vp, kc, vc = W.extend_inputs(500 + P, P, C, hq, hkv)
    w = W.small_workload(501 + P, 1, hq, hkv, [P + C])
    slots = W.slots(w, 0, P, P + C)
    stale = np.full(oracle.pool_bytes(w.num_pages, hkv), 0xA5, dtype=np.uint8)
    gpool = B.Pool(w.num_pages, hkv, device="cuda", data=torch.as_tensor(stale.copy(), device="cuda"))
    sm = 128 ** -0.5
    plain, _ = _run(q, kp, vp, kc, vc, sm)
    out = B.nvfp4_extend_attn(q.cuda(), kp.cuda(), vp.cuda(), kc.cuda(), vc.cuda(), sm, chunk_pool=gpool,
                              chunk_slots=torch.as_tensor(slots, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), plain)
    opool = stale.copy()
    oracle.quantize_to_pool(bf16_bits(kc), bf16_bits(vc), slots, w.num_pages, pool=opool)
    got = gpool.data.cpu().numpy()
    assert np.array_equal(got, opool), f"pool bytes differ at {np.flatnonzero(got != opool)[:8]}"


def test_extend_fused_chunk_write_full_size():
    """Workload 5's 8192-token bf16 chunk written by the extend launch into the
    extend request's pages, checked byte for byte against the oracle."""
    w = W.config(5)
    P, C, hq, hkv = w.extend_prefix, w.extend_chunk, w.num_q_heads, w.num_kv_heads
    print(f"fused write full size P={P} C={C}", flush=True)
    _, kp, vp, _, _ = W.extend_inputs(w.seed, 64, 1, hq, hkv, device="cuda")  # the write does not read the prefix
    kc, vc = W.extend_chunk_kv(w, device="cuda")
    qc = W.extend_query(w, device="cuda")
    slots = W.slots(w, w.extend_row, P, P + C)
    pages = np.unique(slots // 16)
    gpool = B.Pool(w.num_pages, hkv, device="cuda")
    B.nvfp4_extend_attn(qc, kp, vp, kc, vc, w.sm_scale, chunk_pool=gpool,
                        chunk_slots=torch.as_tensor(slots, device="cuda"))
    torch.cuda.synchronize()
    opool = np.zeros(oracle.pool_bytes(w.num_pages, hkv), dtype=np.uint8)
    oracle.quantize_to_pool(bf16_bits(kc), bf16_bits(vc), slots, w.num_pages, pool=opool, n_threads=8)
    slab_pages = torch.as_tensor(pages, device="cuda", dtype=torch.long)
    got = gpool.data.view(w.num_pages, -1)[slab_pages].cpu().numpy()
    ref = opool.reshape(w.num_pages, -1)[pages]
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} bytes differ"


def _untile_v(vt: np.ndarray, rows: int) -> np.ndarray:
    """[tiles, Hkv, 128, 64] f16 tiles (layout of the C header's NVFP4KV_F16_TILED)
    back to rows [rows, Hkv, 128]."""
    tiles, hkv, _, _ = vt.shape
    flat = vt.reshape(tiles, hkv, 128, 8, 2, 4)  # [tile][h][d][unit][half][pos]
    out = np.empty((tiles * 64, hkv, 128), dtype=vt.dtype)
    for k in range(64):
        u, half, pos = 4 * (k // 32) + (k // 4) % 4, (k // 16) % 2, k % 4
        out[k::64] = flat[:, :, :, u, half, pos]
    return out[:rows]


@pytest.mark.parametrize("g", [1.0, float(np.float32(0.3))])
def test_dequant_tiled_workspace_bitexact(g):
    """K as bf16 rows, V as f16 tiles: every value the nearest of its dtype to the
    exact dequantized value (one rounding), rows of the last tile past the prefix
    zero."""
    lens = [37, 200]
    w = W.small_workload(870, 2, 8, 2, lens, name="tiled")
    kv = [(k * g, v * g) for k, v in (W.kv(w, b, 0, L) for b, L in enumerate(lens))]
    gpool = gpu_pool_from_kv(w, kv, g=g)
    opool = oracle_pool_from_kv(w, kv, g=g)
    offs = [0, 64]  # each sequence on its own tiles
    rows = offs[-1] + lens[-1]
    k_ws = torch.full((rows, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_ws = B.tiled_v_workspace(rows, 2)
    v_ws.fill_(float("nan"))
    B.nvfp4_kv_dequant_workspace(gpool, torch.as_tensor(w.page_table, device="cuda"),
                                 torch.as_tensor(w.seq_lens, device="cuda"),
                                 torch.tensor(offs, dtype=torch.int64, device="cuda"), max(lens), k_ws, v_ws)
    torch.cuda.synchronize()
    ko, vo = oracle.dequant_workspace(opool, 2, w.page_table, w.seq_lens, g=g)
    v_rows = _untile_v(v_ws.cpu().numpy(), rows)
    kb = bf16_bits(k_ws)
    cum = np.concatenate([[0], np.cumsum(lens)])
    for s_, (o, L) in enumerate(zip(offs, lens)):
        ref_k, ref_v = ko[cum[s_]:cum[s_] + L], vo[cum[s_]:cum[s_] + L]
        assert np.array_equal(kb[o:o + L], oracle.bf16_bits_of(ref_k)), f"K rows of sequence {s_}"
        want = ref_v.astype(np.float16)  # one rounding from the exact value
        got = v_rows[o:o + L]
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"V of sequence {s_}"
        end = -(-(o + L) // 64) * 64
        pad = _untile_v(v_ws.cpu().numpy(), end)[o + L:end]
        assert np.all(pad == 0), f"padding rows of sequence {s_} not zero"


@pytest.mark.parametrize("offs", [[3, 40, 300], [0, 69, 320]])
def test_dequant_tiled_packed_sequences(offs):
    """Sequences packed into shared tiles: every sequence's K and V rows are
    exact (one rounding), a sequence on a multiple of 64 gets zero rows to the
    end of its last tile, and every other workspace row is left as it was."""
    lens = [37, 200, 50]
    print(f"tiled dequant, row offsets {offs}", flush=True)
    w = W.small_workload(890 + offs[0], 3, 8, 2, lens, name="tiled_packed")
    kv = [W.kv(w, b, 0, L) for b, L in enumerate(lens)]
    gpool = gpu_pool_from_kv(w, kv)
    opool = oracle_pool_from_kv(w, kv)
    rows = 384
    k_ws = torch.full((rows, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_ws = B.tiled_v_workspace(rows, 2)
    v_ws.fill_(float("nan"))
    B.nvfp4_kv_dequant_workspace(gpool, torch.as_tensor(w.page_table, device="cuda"),
                                 torch.as_tensor(w.seq_lens, device="cuda"),
                                 torch.tensor(offs, dtype=torch.int64, device="cuda"), max(lens), k_ws, v_ws)
    torch.cuda.synchronize()
    ko, vo = oracle.dequant_workspace(opool, 2, w.page_table, w.seq_lens)
    v_rows = _untile_v(v_ws.cpu().numpy(), rows)
    kb = bf16_bits(k_ws)
    cum = np.concatenate([[0], np.cumsum(lens)])
    written = np.zeros(rows, dtype=bool)
    zero = np.zeros(rows, dtype=bool)
    for s_, (o, L) in enumerate(zip(offs, lens)):
        assert np.array_equal(kb[o:o + L], oracle.bf16_bits_of(ko[cum[s_]:cum[s_] + L])), f"K rows of sequence {s_}"
        want = vo[cum[s_]:cum[s_] + L].astype(np.float16)
        assert np.array_equal(v_rows[o:o + L].view(np.uint16), want.view(np.uint16)), f"V of sequence {s_}"
        written[o:o + L] = True
        if o % 64 == 0:
            zero[o + L:-(-(o + L) // 64) * 64] = True
    assert np.all(v_rows[zero] == 0), "padding rows of an own-tile sequence not zero"
    untouched = ~(written | zero)
    assert np.all(np.isnan(v_rows[untouched])), "V rows of no sequence were written"
    assert np.all(np.isnan(k_ws.float().cpu().numpy()[untouched | zero])), "K rows of no sequence were written"


@pytest.mark.parametrize("P,C,hq,hkv", [(100, 37, 8, 1), (200, 130, 64, 8), (64, 64, 16, 2)])
def test_extend_over_tiled_workspace(P, C, hq, hkv):
    """Attention over the tiled workspace (V^T tiles copied as they are) equals
    attention over the bf16 workspace of the same pool bit for bit (the f16 V
    values are the same), and the oracle within the bar."""
    print(f"tiled extend P={P} C={C} Hq={hq} Hkv={hkv}", flush=True)
    w = W.small_workload(880 + P, 1, hq, hkv, [P + C])
    k, v = W.kv(w, 0, 0, P + C)
    gpool = gpu_pool_from_kv(w, [(k[:P], v[:P])])
    pt = torch.as_tensor(w.page_table, device="cuda")
    sl = torch.tensor([P], dtype=torch.int32, device="cuda")
    ro = torch.zeros(1, dtype=torch.int64, device="cuda")
    kb = torch.empty((P, hkv, 128), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    B.nvfp4_kv_dequant_workspace(gpool, pt, sl, ro, P, kb, vb)
    vt = B.tiled_v_workspace(P, hkv)
    kt = torch.empty_like(kb)
    B.nvfp4_kv_dequant_workspace(gpool, pt, sl, ro, P, kt, vt)
    q = W.extend_inputs(881 + P, 0, C, hq, hkv)[0]
    kc, vc = k[P:].to(torch.bfloat16), v[P:].to(torch.bfloat16)
    sm = 128 ** -0.5
    lse_a = torch.empty((C, hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    out_b = B.nvfp4_extend_attn(q.cuda(), kb, vb, kc.cuda(), vc.cuda(), sm, lse=lse_b)
    out_t = B.nvfp4_extend_attn(q.cuda(), kt, vt, kc.cuda(), vc.cuda(), sm, lse=lse_a)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out_b) and torch.equal(lse_a, lse_b)
    kp = kb.float().cpu().numpy()
    vp = _untile_v(vt.cpu().numpy(), P).astype(np.float32)
    ref, ref_lse = oracle.extend_attn(bf16_bits(q), kp, vp, bf16_bits(kc), bf16_bits(vc), sm, n_threads=8)
    assert_close(out_t.float().cpu().numpy(), ref, what="tiled extend")
    assert_close(lse_a.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4, what="tiled extend lse")
