"""CPU-side checks of the C-ABI library: it loads, exports every symbol the header
declares, and its host validation rejects bad arguments before any HIP call (no
compute call is made here; device pointers are fake, never dereferenced)."""
import ctypes
import os
import re

import pytest

from bit_paged_kv_nvfp4_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4kv.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_WORKSPACE, ERR_VALUE, ERR_HIP, ERR_SCRATCH = range(9)
FAKE = 0x10000  # 16-byte aligned, never dereferenced by validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*((?:nvfp4|fp8)[a-z_0-9]*)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        import bit_paged_kv_nvfp4_amd.build as bld

        bld.build()
    return B.lib()


def pool(num_pages=4, hkv=1, g=1.0, data=FAKE):
    return B.PoolDesc(data, num_pages, hkv, g)


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert set(decl) == set(B.EXPORTED), decl
    for name in decl:
        assert hasattr(L, name), name


def test_constants_and_strings(L):
    assert L.nvfp4kv_version() == 2
    assert L.nvfp4kv_pool_bytes(10, 8) == 10 * 8 * 2 * 1152
    for s in range(9):
        assert len(B.status_string(s)) > 0
    assert B.status_string(99) == "unknown status"


def test_default_splits_and_workspace_size(L):
    # 256 CUs hold 1024 persistent workgroups; about 16 splits per workgroup window
    # over 44 x 8 (sequence, KV head) segments: ceil(16 * 1024 / 352) = 47
    assert L.nvfp4_paged_decode_attn_default_splits(44, 8, 32768, 256) == 47
    assert L.nvfp4_paged_decode_attn_default_splits(1, 1, 16, 256) == 1
    # a small cache gets at most one workgroup per 8 pages: 1 x 1 x 128 pages -> 16
    # workgroups, 16 * 16 = 256 splits, capped at 4 pages per split -> 32
    assert L.nvfp4_paged_decode_attn_default_splits(1, 1, 2048, 256) == 32
    # 2 x 8 segments of 300 pages -> 600 workgroups (below 1024), 600 splits, capped at 300 / 4 = 75
    assert L.nvfp4_paged_decode_attn_default_splits(2, 8, 4800, 256) == 75
    # 8 x 8 segments of 64 pages -> 512 workgroups, ceil(16 * 512 / 64) = 128, capped at 64 / 4 = 16
    assert L.nvfp4_paged_decode_attn_default_splits(8, 8, 1024, 256) == 16
    assert L.nvfp4_paged_decode_attn_default_splits(2, 8, 1048576, 256) <= 4096
    s = L.nvfp4_paged_decode_attn_default_splits(15, 8, 163840, 256)
    assert 1 <= s <= 163840 // 16 // 4
    ws = L.nvfp4_paged_decode_attn_workspace_bytes(3, 16, 5)
    assert ws >= 3 * 16 * 5 * 130 * 4
    assert L.nvfp4_paged_decode_attn_workspace_bytes(3, 16, 0) == 0
    assert L.nvfp4_paged_decode_attn_workspace_bytes(3, 16, 5000) == 0


def q_call(L, p, k=FAKE, v=FAKE, dt=0, ts=1024, hs=128, slots=FAKE, T=16):
    return L.nvfp4_kv_quantize(k, v, dt, ts, hs, slots, T, ctypes.byref(p) if p is not None else None, None)


def test_quantize_validation(L):
    assert q_call(L, None) == ERR_NULL
    assert q_call(L, pool(data=0)) == ERR_NULL
    assert q_call(L, pool(data=FAKE + 8)) == ERR_ALIGN
    assert q_call(L, pool(num_pages=0)) == ERR_SHAPE
    assert q_call(L, pool(hkv=0)) == ERR_SHAPE
    assert q_call(L, pool(g=3.0), T=0) == OK  # any finite g in [2^-64, 2^64]
    assert q_call(L, pool(g=0.0)) == ERR_VALUE
    assert q_call(L, pool(g=-0.3)) == ERR_VALUE
    assert q_call(L, pool(g=2.0 ** -70)) == ERR_VALUE
    assert q_call(L, pool(g=float("nan"))) == ERR_VALUE
    assert q_call(L, pool(g=2.0 ** 70)) == ERR_VALUE
    assert q_call(L, pool(), dt=2) == ERR_DTYPE
    assert q_call(L, pool(), T=-1) == ERR_SHAPE
    assert q_call(L, pool(), T=0) == OK  # no-op, no HIP call
    assert q_call(L, pool(), k=None) == ERR_NULL
    assert q_call(L, pool(), slots=None) == ERR_NULL
    assert q_call(L, pool(), k=FAKE + 4) == ERR_ALIGN
    assert q_call(L, pool(), ts=1026) == ERR_ALIGN
    assert q_call(L, pool(), dt=1, hs=132) == ERR_ALIGN
    assert q_call(L, pool(), slots=FAKE + 2) == ERR_ALIGN


def d_call(L, p, q=FAKE, pt=FAKE, stride=8, sl=FAKE, B_=2, hq=8, maxlen=100, sm=0.088, splits=2, ws=FAKE,
           wsb=1 << 30, out=FAKE, odt=1, lse=None):
    return L.nvfp4_paged_decode_attn(q, pt, stride, sl, B_, hq, maxlen, ctypes.byref(p) if p is not None else None,
                                     sm, splits, ws, wsb, out, odt, lse, None)


def test_decode_validation(L):
    assert d_call(L, None) == ERR_NULL
    assert d_call(L, pool(g=float("inf"))) == ERR_VALUE
    assert d_call(L, pool(g=0.3), B_=0) == OK
    assert d_call(L, pool(), odt=2) == ERR_DTYPE
    assert d_call(L, pool(), B_=-1) == ERR_SHAPE
    assert d_call(L, pool(), hq=0) == ERR_SHAPE
    assert d_call(L, pool(hkv=3), hq=8) == ERR_SHAPE  # 8 % 3
    assert d_call(L, pool(hkv=1), hq=17) == ERR_SHAPE  # group > 16
    assert d_call(L, pool(), maxlen=8 * 16 + 1) == ERR_SHAPE  # beyond the page-table row
    assert d_call(L, pool(), splits=4097) == ERR_SHAPE
    assert d_call(L, pool(), splits=-1) == ERR_SHAPE
    assert d_call(L, pool(), sm=float("inf")) == ERR_VALUE
    assert d_call(L, pool(), B_=0) == OK  # no-op, no HIP call
    assert d_call(L, pool(), q=None) == ERR_NULL
    assert d_call(L, pool(), ws=None) == ERR_NULL
    assert d_call(L, pool(), out=None) == ERR_NULL
    assert d_call(L, pool(), q=FAKE + 2) == ERR_ALIGN
    assert d_call(L, pool(), out=FAKE + 4) == ERR_ALIGN
    assert d_call(L, pool(), lse=FAKE + 1) == ERR_ALIGN
    need = L.nvfp4_paged_decode_attn_workspace_bytes(2, 8, 2)
    assert d_call(L, pool(), wsb=need - 1) == ERR_WORKSPACE


def x_call(L, p, pt=FAKE, stride=8, sl=FAKE, ro=FAKE, n=2, maxlen=64, k=FAKE, v=FAKE, odt=1):
    return L.nvfp4_kv_dequant_workspace(ctypes.byref(p) if p is not None else None, pt, stride, sl, ro, n, maxlen,
                                        k, v, odt, None)


def test_dequant_validation(L):
    assert x_call(L, None) == ERR_NULL
    assert x_call(L, pool(g=-1.0)) == ERR_VALUE
    assert x_call(L, pool(), odt=5) == ERR_DTYPE
    assert x_call(L, pool(), n=-1) == ERR_SHAPE
    assert x_call(L, pool(), maxlen=8 * 16 + 1) == ERR_SHAPE
    assert x_call(L, pool(), n=0) == OK
    assert x_call(L, pool(), maxlen=0) == OK
    assert x_call(L, pool(), ro=None) == ERR_NULL
    assert x_call(L, pool(), k=FAKE + 2) == ERR_ALIGN
    assert x_call(L, pool(), ro=FAKE + 4) == ERR_ALIGN


def e_call(L, q=FAKE, kp=FAKE, vp=FAKE, pdt=1, P=100, kc=FAKE, vc=FAKE, C=10, hq=8, hkv=1, sm=0.088, out=FAKE,
           lse=None):
    return L.nvfp4_extend_attn(q, kp, vp, pdt, P, kc, vc, C, hq, hkv, sm, 0.0, out, lse, None, None, None)


def test_extend_validation(L):
    assert e_call(L, pdt=0) == ERR_DTYPE  # f32 prefix is not an attention input
    assert e_call(L, pdt=7) == ERR_DTYPE
    assert e_call(L, P=-1) == ERR_SHAPE
    assert e_call(L, C=-1) == ERR_SHAPE
    assert e_call(L, hq=0) == ERR_SHAPE
    assert e_call(L, hq=8, hkv=3) == ERR_SHAPE
    assert e_call(L, hq=17, hkv=1) == ERR_SHAPE  # group > 16
    assert e_call(L, sm=float("nan")) == ERR_VALUE
    assert e_call(L, C=0) == OK  # no-op, no HIP call
    assert e_call(L, q=None) == ERR_NULL
    assert e_call(L, kc=None) == ERR_NULL
    assert e_call(L, out=None) == ERR_NULL
    assert e_call(L, kp=None) == ERR_NULL
    assert e_call(L, q=FAKE + 2) == ERR_ALIGN
    assert e_call(L, vp=FAKE + 8) == ERR_ALIGN
    assert e_call(L, lse=FAKE + 2) == ERR_ALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def fp8_pool(num_pages=4, hkv=1, ks=1.0, vs=1.0, data=FAKE):
    return B.Fp8PoolDesc(data, num_pages, hkv, ks, vs)


def test_fp8_baseline_validation(L):
    assert L.fp8kv_pool_bytes(10, 8) == 10 * 8 * 2 * 2048
    assert L.fp8_paged_decode_attn_default_splits(44, 8, 32768, 256) == 47
    q = lambda p, **kw: L.fp8_kv_quantize(kw.get("k", FAKE), FAKE, kw.get("dt", 0), 1024, 128, FAKE, kw.get("T", 16),
                                          ctypes.byref(p) if p is not None else None, None)
    assert q(None) == ERR_NULL
    assert q(fp8_pool(data=0)) == ERR_NULL
    assert q(fp8_pool(ks=3.0)) == ERR_VALUE
    assert q(fp8_pool(vs=0.0)) == ERR_VALUE
    assert q(fp8_pool(hkv=0)) == ERR_SHAPE
    assert q(fp8_pool(), dt=2) == ERR_DTYPE
    assert q(fp8_pool(), T=0) == OK
    assert q(fp8_pool(), k=FAKE + 4) == ERR_ALIGN
    d = lambda p, **kw: L.fp8_paged_decode_attn(FAKE, FAKE, 8, FAKE, kw.get("B", 2), kw.get("hq", 8), 100,
                                                ctypes.byref(p) if p is not None else None, 0.088, 2, FAKE, 1 << 30,
                                                FAKE, kw.get("odt", 1), None, None)
    assert d(None) == ERR_NULL
    assert d(fp8_pool(vs=0.75)) == ERR_VALUE
    assert d(fp8_pool(), odt=2) == ERR_DTYPE
    assert d(fp8_pool(hkv=3), hq=8) == ERR_SHAPE
    assert d(fp8_pool(), B=0) == OK


def test_global_scale_rule_matches_oracle(L):
    import numpy as np

    import oracle

    rng = np.random.default_rng(81)
    for a in list(np.exp(rng.uniform(np.log(1e-8), np.log(1e12), 400)).astype(np.float32)) + [0.0, 2688.0, 1344.0]:
        g = B.nvfp4kv_global_scale_for_amax(float(a))
        assert g == oracle.global_scale_for_amax(float(a)), a
    assert B.nvfp4kv_global_scale_for_amax(float("nan")) == 0.0
    assert B.nvfp4kv_global_scale_for_amax(-1.0) == 0.0
    assert B.nvfp4kv_global_scale_for_amax(3e38) == 0.0  # g beyond 2^64


def test_amax_validation(L):
    ws_need = L.nvfp4_kv_amax_workspace_bytes()
    assert ws_need == 256 * 2 * 4
    a = lambda **kw: L.nvfp4_kv_amax(kw.get("k", FAKE), FAKE, kw.get("dt", 0), kw.get("ts", 1024), 128,
                                     kw.get("T", 16), kw.get("hkv", 8), kw.get("out", FAKE), kw.get("ws", FAKE),
                                     kw.get("wsb", ws_need), None)
    assert a(dt=2) == ERR_DTYPE
    assert a(T=-1) == ERR_SHAPE
    assert a(hkv=0) == ERR_SHAPE
    assert a(out=None) == ERR_NULL
    assert a(ws=None) == ERR_NULL
    assert a(k=None) == ERR_NULL
    assert a(wsb=ws_need - 1) == ERR_WORKSPACE
    assert a(k=FAKE + 4) == ERR_ALIGN
    assert a(ts=1026) == ERR_ALIGN
    assert a(out=FAKE + 2) == ERR_ALIGN


def test_extend_fused_write_validation(L):
    p = pool(hkv=1)
    call = lambda pl, slots: L.nvfp4_extend_attn(FAKE, FAKE, FAKE, 1, 100, FAKE, FAKE, 10, 8, 1, 0.088, 0.0, FAKE, None,
                                                 ctypes.byref(pl) if pl is not None else None, slots, None)
    assert call(pool(hkv=2), FAKE) == ERR_SHAPE  # pool heads differ
    assert call(pool(g=2.0 ** 65, hkv=1), FAKE) == ERR_VALUE
    assert call(p, None) == ERR_NULL
    assert call(p, FAKE + 2) == ERR_ALIGN


def test_decode_append_validation(L):
    """The fused decode step checks its new rows (as the quantize call checks its
    sources) after the decode arguments, all before any HIP call."""
    def a(fn, p, **kw):
        return fn(FAKE, kw.get("k", FAKE), kw.get("v", FAKE), kw.get("dt", 1), kw.get("ts", 1024), kw.get("hs", 128),
                  FAKE, 8, FAKE, kw.get("B", 2), kw.get("hq", 8), 100, ctypes.byref(p) if p is not None else None,
                  0.088, 2, FAKE, 1 << 30, kw.get("out", FAKE), kw.get("odt", 1), kw.get("lse"), None)

    for fn, good, bad_scale in ((L.nvfp4_paged_decode_attn_append, pool(hkv=2), pool(hkv=2, g=0.0)),
                                (L.fp8_paged_decode_attn_append, fp8_pool(hkv=2), fp8_pool(hkv=2, ks=3.0))):
        assert a(fn, None) == ERR_NULL
        assert a(fn, bad_scale) == ERR_VALUE
        assert a(fn, good, odt=2) == ERR_DTYPE
        assert a(fn, good, hq=7) == ERR_SHAPE
        assert a(fn, good, k=None) == ERR_NULL
        assert a(fn, good, v=None) == ERR_NULL
        assert a(fn, good, dt=2) == ERR_DTYPE
        assert a(fn, good, ts=-8) == ERR_SHAPE
        assert a(fn, good, k=FAKE + 4) == ERR_ALIGN
        assert a(fn, good, hs=4) == ERR_ALIGN  # bf16 rows need multiples of 8 elements
        assert a(fn, good, B=0) == OK  # no-op, no HIP call
        assert a(fn, good, B=0, k=None) == OK
        assert a(fn, good, out=None, lse=FAKE) == ERR_NULL  # lse needs the combine
        assert a(fn, good, out=None, B=0) == OK  # phase 1 only, nothing to do


# ---- argument checks of the Python binding (raised before any library call) ----
def _decode_args(batch=3, hq=16, hkv=2, stride=4):
    import torch

    p = B.Pool(8, hkv, device="cpu")
    q = torch.zeros((batch, hq, 128), dtype=torch.bfloat16)
    pt = torch.zeros((batch, stride), dtype=torch.int32)
    sl = torch.full((batch,), 16, dtype=torch.int32)
    return q, pt, sl, p


def test_binding_rejects_int64_seq_lens(L):
    import torch

    q, pt, sl, p = _decode_args()
    # int64 lengths would be read by the kernel as int32 pairs [L0, 0, L1, 0, ...]
    with pytest.raises(ValueError, match="seq_lens"):
        B.nvfp4_paged_decode_attn(q, pt, sl.to(torch.int64), p, 0.1, 16)
    with pytest.raises(ValueError, match="seq_lens"):
        B.nvfp4_paged_decode_attn(q, pt, sl[:2], p, 0.1, 16)
    with pytest.raises(ValueError, match="seq_lens"):
        B.nvfp4_paged_decode_attn_partial(q, pt, sl.to(torch.int64), p, 0.1, 16, 1, torch.zeros(16, dtype=torch.uint8))


def test_binding_rejects_short_outputs(L):
    import torch

    q, pt, sl, p = _decode_args()
    short = torch.zeros((2, 16, 128), dtype=torch.float32)  # batch 3 needs [3, 16, 128]
    with pytest.raises(ValueError, match="out must be"):
        B.nvfp4_paged_decode_attn(q, pt, sl, p, 0.1, 16, out=short)
    with pytest.raises(ValueError, match="lse must be"):
        B.nvfp4_paged_decode_attn(q, pt, sl, p, 0.1, 16, lse=torch.zeros((3, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="lse must be"):
        B.nvfp4_paged_decode_attn(q, pt, sl, p, 0.1, 16, lse=torch.zeros((3, 16), dtype=torch.float64))
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out must be"):
        B.nvfp4_decode_combine(ws, 3, 16, 1, short)


def test_binding_rejects_bad_query_and_table(L):
    import torch

    q, pt, sl, p = _decode_args()
    with pytest.raises(ValueError, match="q must be"):
        B.nvfp4_paged_decode_attn(torch.zeros((3, 16, 64), dtype=torch.bfloat16), pt, sl, p, 0.1, 16)
    with pytest.raises(ValueError, match="multiple"):
        B.nvfp4_paged_decode_attn(torch.zeros((3, 15, 128), dtype=torch.bfloat16), pt, sl, p, 0.1, 16)
    with pytest.raises(ValueError, match="page_table has 2 rows"):
        B.nvfp4_paged_decode_attn(q, pt[:2], sl, p, 0.1, 16)
    with pytest.raises(ValueError, match="max_seq_len"):
        B.nvfp4_paged_decode_attn(q, pt, sl, p, 0.1, 4 * 16 + 1)
    kn = torch.zeros((3, 2, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="seq_lens"):
        B.nvfp4_paged_decode_attn_append(q, kn, kn, pt, sl.to(torch.int64), p, 0.1, 16)


def test_binding_rejects_bad_extend_and_dequant_shapes(L):
    import torch

    p = B.Pool(8, 2, device="cpu")
    pt = torch.zeros((2, 4), dtype=torch.int32)
    sl = torch.full((2,), 16, dtype=torch.int32)
    ro = torch.zeros(2, dtype=torch.int64)
    ko = torch.zeros((32, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="row_offsets"):
        B.nvfp4_kv_dequant_workspace(p, pt, sl, ro[:1], 16, ko, ko.clone())
    with pytest.raises(ValueError, match="k_out must be"):
        B.nvfp4_kv_dequant_workspace(p, pt, sl, ro, 16, torch.zeros((32, 3, 128), dtype=torch.bfloat16),
                                     torch.zeros((32, 3, 128), dtype=torch.bfloat16))
    q = torch.zeros((5, 4, 128), dtype=torch.bfloat16)
    kp = torch.zeros((7, 2, 128), dtype=torch.bfloat16)
    kc = torch.zeros((5, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_chunk and v_chunk"):
        B.nvfp4_extend_attn(q, kp, kp, kc[:4], kc[:4], 0.1)
    with pytest.raises(ValueError, match="out must be"):
        B.nvfp4_extend_attn(q, kp, kp, kc, kc, 0.1, out=torch.zeros((4, 4, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must be"):
        B.nvfp4_extend_attn(q, kp, kp, kc, kc, 0.1, lse=torch.zeros((5, 2), dtype=torch.float32))


def test_noalloc_decode_rejects_before_any_hip_call(L):
    P = B.PoolDesc(FAKE, 4096, 8, 1.0)
    fn = L.nvfp4_paged_decode_attn_noalloc
    common = (FAKE, FAKE, 4096, FAKE, 44, 64, 32768)
    # 44 x 64 x 47 splits need 69 MB of states, more than the 64 MiB scratch
    assert fn(*common, ctypes.byref(P), 0.1, 47, FAKE, 1, None, None) == ERR_SCRATCH
    # so many (sequence, head) rows that even one split does not fit
    assert fn(FAKE, FAKE, 4096, FAKE, 1 << 20, 64, 32768, ctypes.byref(P), 0.1, 1, FAKE, 1, None, None) == ERR_SCRATCH
    assert fn(*common, ctypes.byref(P), 0.1, 8, FAKE, 7, None, None) == ERR_DTYPE
    assert fn(*common, ctypes.byref(P), 0.1, 5000, FAKE, 1, None, None) == ERR_SHAPE
    assert fn(FAKE, FAKE, 4096, FAKE, 44, 60, 32768, ctypes.byref(P), 0.1, 8, FAKE, 1, None, None) == ERR_SHAPE
    assert fn(*common, ctypes.byref(P), float("nan"), 8, FAKE, 1, None, None) == ERR_VALUE
    assert fn(*common, ctypes.byref(P), 0.1, 8, None, 1, None, None) == ERR_NULL
    assert fn(*common, ctypes.byref(P), 0.1, 8, FAKE + 4, 1, None, None) == ERR_ALIGN
    assert fn(FAKE, FAKE, 4096, FAKE, 0, 64, 32768, ctypes.byref(P), 0.1, 8, FAKE, 1, None, None) == OK
    assert L.nvfp4_paged_decode_attn_workspace_bytes(44, 64, 47) > (64 << 20)


def test_tight_global_scale_matches_oracle(L):
    import numpy as np

    import oracle

    rng = np.random.default_rng(5)
    for a in np.float32(np.exp(rng.uniform(np.log(1e-9), np.log(1e12), 2000))):
        assert B.nvfp4kv_global_scale_tight_for_amax(float(a)) == oracle.global_scale_tight_for_amax(float(a)), a
    assert B.nvfp4kv_global_scale_tight_for_amax(0.0) == 1.0
    assert B.nvfp4kv_global_scale_tight_for_amax(float("inf")) == 0.0
    assert B.nvfp4kv_global_scale_tight_for_amax(-2.0) == 0.0


def test_extend_v_bound_validation(L):
    call = lambda vb: L.nvfp4_extend_attn(FAKE, FAKE, FAKE, 1, 100, FAKE, FAKE, 0, 8, 1, 0.088, vb, FAKE, None, None,
                                          None, None)
    assert call(0.0) == OK and call(1e30) == OK  # C = 0: nothing to do
    assert call(-1.0) == ERR_VALUE
    assert call(float("nan")) == ERR_VALUE
    assert call(float("inf")) == ERR_VALUE


def test_host_page_table_check(L):
    import numpy as np

    from bit_paged_kv_nvfp4_amd import workload as W

    w = W.small_workload(3, 4, 8, 1, [40, 16, 0, 33])
    B.nvfp4kv_check_page_table(w.page_table, w.seq_lens, w.max_seq_len, w.num_pages, exclusive=True)
    bad = w.page_table.copy()
    bad[1, 0] = w.num_pages  # outside the pool
    with pytest.raises(ValueError, match=r"page_table\[1\]\[0\]"):
        B.nvfp4kv_check_page_table(bad, w.seq_lens, w.max_seq_len, w.num_pages)
    bad = w.page_table.copy()
    bad[3, 2] = -1
    with pytest.raises(ValueError, match=r"page_table\[3\]\[2\]"):
        B.nvfp4kv_check_page_table(bad, w.seq_lens, w.max_seq_len, w.num_pages)
    # entries past a sequence's last page are not read, so they are not checked
    ok = w.page_table.copy()
    ok[1, 1:] = 10 ** 6
    B.nvfp4kv_check_page_table(ok, w.seq_lens, w.max_seq_len, w.num_pages)
    lens = w.seq_lens.copy()
    lens[0] = 41  # beyond max_seq_len 40
    with pytest.raises(ValueError, match=r"seq_lens\[0\]"):
        B.nvfp4kv_check_page_table(w.page_table, lens, 40, w.num_pages)
    lens = w.seq_lens.copy()
    lens[2] = -1
    with pytest.raises(ValueError, match=r"seq_lens\[2\]"):
        B.nvfp4kv_check_page_table(w.page_table, lens, w.max_seq_len, w.num_pages)
    with pytest.raises(ValueError, match=r"seq_lens\[0\]"):  # more tokens than the row has pages
        B.nvfp4kv_check_page_table(w.page_table, np.array([16 * w.page_table.shape[1] + 1, 0, 0, 0]), 10 ** 6,
                                   w.num_pages)
    shared = w.page_table.copy()
    shared[3, 1] = shared[0, 2]  # one physical page in two sequences
    B.nvfp4kv_check_page_table(shared, w.seq_lens, w.max_seq_len, w.num_pages)  # fine without exclusive
    with pytest.raises(ValueError, match=r"page_table\[3\]\[1\].*already holds"):
        B.nvfp4kv_check_page_table(shared, w.seq_lens, w.max_seq_len, w.num_pages, exclusive=True)
    # the C entry point's own argument checks
    assert L.nvfp4kv_check_page_table(None, 4, None, 0, 0, 1, None, None) == OK
    assert L.nvfp4kv_check_page_table(None, 4, FAKE, 1, 0, 1, None, None) == ERR_NULL
    assert L.nvfp4kv_check_page_table(FAKE, 0, FAKE, 1, 0, 1, None, None) == ERR_SHAPE
