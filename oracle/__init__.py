"""CPU oracle for NVFP4 paged-KV decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``nvfp4kv_oracle.c`` (plain
scalar C, fp64 arithmetic, built with gcc) through ctypes and shares no code
with the GPU library. See the C file's header for what each step computes and
which page and section it follows.

Parity status of each function (what pins it is listed in the tests):
  e2m1_value, e4m3_value           pinned (closed form; library float8 decoder)
  scale_byte, e2m1_code,
  quantize_block16                 pinned (exact-rational brute force; library
                                   RNE conversion; worked example; round trip)
  quantize_to_pool, dequant_row,
  dequant_workspace                pinned (round trip of representable blocks
                                   through a permuted page table)
  decode_attn                      pinned (fp64 library SDPA on representable
                                   K/V; closed-form special cases)
  fp8_* (FP8 baseline pool)        pinned (codes vs library float8 cast of x/s;
                                   layout bijection; attention vs fp64 SDPA on
                                   E4M3-representable K/V with scales)
  amax, global_scale_for_amax,
  global_scale_tight_for_amax      pinned (library max; closed forms and
                                   minimality over powers of two / binary32)
  bf16_bits_of                     pinned (library RNE cast of float32-exact
                                   values; exact-rational nearest-even)
  any finite global scale g        pinned (exact-rational brute force of scale
                                   and codes at non-power-of-two g, threshold
                                   sweeps +-1 ulp, exact dequantized products)
  extend_attn                      pinned (fp64 library SDPA with an explicit
                                   prefix + causal mask, all three workspace
                                   dtypes; single-row and equal-key closed forms)
  quantized-vs-unquantized error   parity unpinned (the pages give no number)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4kv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_nvfp4kv.so")

HEAD_DIM = 128
PAGE_SIZE = 16
SLAB_BYTES = 1152


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    c = ctypes
    P = c.c_void_p
    L.orc_e2m1_value.argtypes = [c.c_int]
    L.orc_e2m1_value.restype = c.c_double
    L.orc_e4m3_value.argtypes = [c.c_int]
    L.orc_e4m3_value.restype = c.c_double
    L.orc_scale_byte.argtypes = [c.c_float, c.c_float]
    L.orc_scale_byte.restype = c.c_int
    L.orc_e2m1_code.argtypes = [c.c_float, c.c_double]
    L.orc_e2m1_code.restype = c.c_int
    L.orc_quantize_block16.argtypes = [P, c.c_float, P, P]
    L.orc_quantize_block16.restype = None
    L.orc_slab_offset.argtypes = [c.c_int64, c.c_int, c.c_int, c.c_int]
    L.orc_slab_offset.restype = c.c_int64
    L.orc_e4m3_code_of.argtypes = [c.c_double]
    L.orc_e4m3_code_of.restype = c.c_int
    L.orc_code_nibble.argtypes = [c.c_int, c.c_int, c.c_int]
    L.orc_code_nibble.restype = c.c_int
    L.orc_scale_byte_offset.argtypes = [c.c_int, c.c_int, c.c_int]
    L.orc_scale_byte_offset.restype = c.c_int
    L.orc_pool_bytes.argtypes = [c.c_int64, c.c_int]
    L.orc_pool_bytes.restype = c.c_int64
    L.orc_quantize_to_pool.argtypes = [P, P, c.c_int, c.c_int64, c.c_int64, P, c.c_int64, c.c_int, c.c_float, P,
                                       c.c_int]
    L.orc_quantize_to_pool.restype = None
    L.orc_dequant_row.argtypes = [P, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int, c.c_float, P]
    L.orc_dequant_row.restype = None
    L.orc_dequant_workspace.argtypes = [P, c.c_int, c.c_float, P, c.c_int64, P, P, c.c_int, P, P]
    L.orc_dequant_workspace.restype = None
    L.orc_decode_attn.argtypes = [P, P, c.c_int64, P, c.c_int, c.c_int, c.c_int, P, c.c_float, c.c_double, P,
                                  P, P, c.c_int, c.c_int]
    L.orc_decode_attn.restype = None
    L.orc_extend_attn.argtypes = [P, P, P, c.c_int, c.c_int64, P, P, c.c_int64, c.c_int, c.c_int, c.c_double, P, P,
                                  P, c.c_int64, c.c_int]
    L.orc_extend_attn.restype = None
    L.orc_fp8_slab_offset.argtypes = [c.c_int64, c.c_int, c.c_int, c.c_int]
    L.orc_fp8_slab_offset.restype = c.c_int64
    L.orc_fp8_byte_offset.argtypes = [c.c_int, c.c_int, c.c_int]
    L.orc_fp8_byte_offset.restype = c.c_int
    L.orc_fp8_pool_bytes.argtypes = [c.c_int64, c.c_int]
    L.orc_fp8_pool_bytes.restype = c.c_int64
    L.orc_fp8_code.argtypes = [c.c_float, c.c_float]
    L.orc_fp8_code.restype = c.c_int
    L.orc_fp8_quantize_to_pool.argtypes = [P, P, c.c_int, c.c_int64, c.c_int64, P, c.c_int64, c.c_int, c.c_float,
                                           c.c_float, P]
    L.orc_fp8_quantize_to_pool.restype = None
    L.orc_fp8_dequant_row.argtypes = [P, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int, c.c_float, P]
    L.orc_fp8_dequant_row.restype = None
    L.orc_fp8_decode_attn.argtypes = [P, P, c.c_int64, P, c.c_int, c.c_int, c.c_int, P, c.c_float, c.c_float,
                                      c.c_double, P, P, P, c.c_int, c.c_int]
    L.orc_fp8_decode_attn.restype = None
    L.orc_amax.argtypes = [P, c.c_int, c.c_int64, c.c_int64, c.c_int64, c.c_int]
    L.orc_amax.restype = c.c_double
    L.orc_global_scale_for_amax.argtypes = [c.c_double]
    L.orc_global_scale_for_amax.restype = c.c_double
    L.orc_global_scale_tight_for_amax.argtypes = [c.c_double]
    L.orc_global_scale_tight_for_amax.restype = c.c_float
    L.orc_bf16_bits_of.argtypes = [c.c_double]
    L.orc_bf16_bits_of.restype = c.c_uint16
    L.orc_bf16_bits_of_array.argtypes = [P, c.c_int64, P]
    L.orc_bf16_bits_of_array.restype = None
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = _load(_LIB)
    return _lib


class use_library:
    """Context manager: route every oracle call through another build of the
    oracle source (used by the mutation tests that plant mistakes in it)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def build_variant(source_text: str, out_path: str) -> str:
    """Compile a modified copy of the oracle source (for mutation tests)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", "-O1", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-ffp-contract=off", "-o",
                    out_path, src, "-lm", "-lpthread"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def e4m3_code_of(x: float) -> int:
    """FP8 E4M3 code of a finite value: nearest, ties to even, saturating at 448."""
    return int(lib().orc_e4m3_code_of(float(x)))


def e4m3_codes_of(values: np.ndarray) -> np.ndarray:
    """Elementwise e4m3_code_of over an array (uint8 codes, same shape)."""
    flat = np.asarray(values, dtype=np.float64).ravel()
    f = lib().orc_e4m3_code_of
    return np.fromiter((f(float(v)) for v in flat), dtype=np.uint8, count=flat.size).reshape(np.shape(values))


def code_nibble(kind: int, row: int, channel: int) -> int:
    """Place of the code of (row, channel) in a slab: 2 * byte + (1 for the high nibble)."""
    return int(lib().orc_code_nibble(int(kind), int(row), int(channel)))


def scale_byte_offset(kind: int, row: int, block: int) -> int:
    return int(lib().orc_scale_byte_offset(int(kind), int(row), int(block)))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---- scalar format functions ---------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(int(byte))


def scale_byte(amax: float, g: float = 1.0) -> int:
    return lib().orc_scale_byte(float(amax), float(g))


def e2m1_code(x: float, divisor: float) -> int:
    return lib().orc_e2m1_code(float(x), float(divisor))


def quantize_block16(x, g: float = 1.0):
    """16 float32 values -> (8 packed code bytes as np.uint8[8], scale byte)."""
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(16))
    codes = np.zeros(8, dtype=np.uint8)
    s = np.zeros(1, dtype=np.uint8)
    lib().orc_quantize_block16(_ptr(xa), float(g), _ptr(codes), _ptr(s))
    return codes, int(s[0])


def pool_bytes(num_pages: int, num_kv_heads: int) -> int:
    return int(lib().orc_pool_bytes(int(num_pages), int(num_kv_heads)))


def slab_offset(page: int, head: int, kind: int, num_kv_heads: int) -> int:
    return int(lib().orc_slab_offset(int(page), int(head), int(kind), int(num_kv_heads)))


# ---- pool-level functions --------------------------------------------------
def quantize_to_pool(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, num_pages: int,
                     g: float = 1.0, pool: np.ndarray | None = None, n_threads: int = 1) -> np.ndarray:
    """K, V: [T, Hkv, 128] float32 or bf16 bits (np.uint16). Returns/updates a
    uint8 pool of num_pages pages."""
    assert k.shape == v.shape and k.ndim == 3 and k.shape[2] == HEAD_DIM
    T, hkv, _ = k.shape
    if k.dtype == np.float32:
        dt = 0
    elif k.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("K/V must be float32 or bf16 bits (uint16)")
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v.astype(k.dtype, copy=False))
    sm = np.ascontiguousarray(slot_mapping.astype(np.int32, copy=False))
    if pool is None:
        pool = np.zeros(pool_bytes(num_pages, hkv), dtype=np.uint8)
    assert pool.nbytes == pool_bytes(num_pages, hkv)
    lib().orc_quantize_to_pool(_ptr(k), _ptr(v), dt, hkv * HEAD_DIM, HEAD_DIM, _ptr(sm), T, hkv,
                               float(g), _ptr(pool), int(n_threads))
    return pool


def dequant_row(pool: np.ndarray, page: int, row: int, head: int, kind: int, num_kv_heads: int,
                g: float = 1.0) -> np.ndarray:
    out = np.zeros(HEAD_DIM, dtype=np.float64)
    lib().orc_dequant_row(_ptr(pool), int(page), int(row), int(head), int(kind), int(num_kv_heads),
                          float(g), _ptr(out))
    return out


def dequant_workspace(pool: np.ndarray, num_kv_heads: int, page_table: np.ndarray, seq_lens: np.ndarray,
                      g: float = 1.0):
    """Dense fp64 K^, V^ [sum(seq_lens), Hkv, 128] of the listed sequences."""
    pt = np.ascontiguousarray(page_table.astype(np.int32, copy=False))
    sl = np.ascontiguousarray(seq_lens.astype(np.int32, copy=False))
    cu = np.zeros(len(sl) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(sl)
    rows = int(cu[-1])
    ko = np.zeros((rows, num_kv_heads, HEAD_DIM), dtype=np.float64)
    vo = np.zeros_like(ko)
    lib().orc_dequant_workspace(_ptr(pool), int(num_kv_heads), float(g), _ptr(pt), pt.shape[1], _ptr(sl),
                                _ptr(cu), len(sl), _ptr(ko), _ptr(vo))
    return ko, vo


def decode_attn(q_bf16_bits: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray, pool: np.ndarray,
                num_kv_heads: int, sm_scale: float, g: float = 1.0, units=None, n_threads: int = 1):
    """q: [B, Hq, 128] bf16 bits (uint16). Returns (out fp64 [B,Hq,128], lse fp64 [B,Hq]).
    ``units``: optional iterable of b*Hq + qh to compute (others stay NaN)."""
    q = np.ascontiguousarray(q_bf16_bits.astype(np.uint16, copy=False))
    B, hq, d = q.shape
    assert d == HEAD_DIM and hq % num_kv_heads == 0
    pt = np.ascontiguousarray(page_table.astype(np.int32, copy=False))
    sl = np.ascontiguousarray(seq_lens.astype(np.int32, copy=False))
    out = np.full((B, hq, HEAD_DIM), np.nan, dtype=np.float64)
    lse = np.full((B, hq), np.nan, dtype=np.float64)
    if units is None:
        u_arr, n_u, u_ptr = None, B * hq, None
    else:
        u_arr = np.ascontiguousarray(np.asarray(list(units), dtype=np.int32))
        n_u, u_ptr = len(u_arr), _ptr(u_arr)
    lib().orc_decode_attn(_ptr(q), _ptr(pt), pt.shape[1], _ptr(sl), B, hq, num_kv_heads, _ptr(pool), float(g),
                          float(sm_scale), _ptr(out), _ptr(lse), u_ptr, n_u, int(n_threads))
    return out, lse


_WS_DTYPES = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.uint8): 2}


def extend_attn(q_bf16_bits: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray, k_chunk_bits: np.ndarray,
                v_chunk_bits: np.ndarray, sm_scale: float, units=None, n_threads: int = 1):
    """Extend attention of a C-token chunk after a P-token prefix workspace.
    q: [C, Hq, 128] bf16 bits; k/v_prefix: [P, Hkv, 128] as float32 values,
    uint16 bf16 bits or uint8 FP8 E4M3 bytes; k/v_chunk: [C, Hkv, 128] bf16 bits.
    Returns (out fp64 [C, Hq, 128], lse fp64 [C, Hq]); ``units``: optional
    iterable of i*Hq + qh to compute (others stay NaN)."""
    q = np.ascontiguousarray(q_bf16_bits.astype(np.uint16, copy=False))
    C, hq, d = q.shape
    kp = np.ascontiguousarray(k_prefix)
    vp = np.ascontiguousarray(v_prefix)
    assert kp.dtype == vp.dtype and kp.dtype in _WS_DTYPES and kp.shape == vp.shape
    P, hkv, d2 = kp.shape
    assert d == d2 == HEAD_DIM and hq % hkv == 0
    kc = np.ascontiguousarray(k_chunk_bits.astype(np.uint16, copy=False))
    vc = np.ascontiguousarray(v_chunk_bits.astype(np.uint16, copy=False))
    assert kc.shape == vc.shape == (C, hkv, HEAD_DIM)
    out = np.full((C, hq, HEAD_DIM), np.nan, dtype=np.float64)
    lse = np.full((C, hq), np.nan, dtype=np.float64)
    if units is None:
        u_ptr, n_u = None, C * hq
    else:
        u_arr = np.ascontiguousarray(np.asarray(list(units), dtype=np.int64))
        u_ptr, n_u = _ptr(u_arr), len(u_arr)
    lib().orc_extend_attn(_ptr(q), _ptr(kp) if P else None, _ptr(vp) if P else None, _WS_DTYPES[kp.dtype], P,
                          _ptr(kc), _ptr(vc), C, hq, hkv, float(sm_scale), _ptr(out), _ptr(lse), u_ptr, n_u,
                          int(n_threads))
    return out, lse


# ---- FP8 baseline (E4M3 per value, per-tensor scale) ------------------------
FP8_SLAB_BYTES = 2048


def fp8_pool_bytes(num_pages: int, num_kv_heads: int) -> int:
    return int(lib().orc_fp8_pool_bytes(num_pages, num_kv_heads))


def fp8_byte_offset(kind: int, row: int, channel: int) -> int:
    return int(lib().orc_fp8_byte_offset(kind, row, channel))


def fp8_slab_offset(page: int, head: int, kind: int, num_kv_heads: int) -> int:
    return int(lib().orc_fp8_slab_offset(page, head, kind, num_kv_heads))


def fp8_code(x: float, scale: float = 1.0) -> int:
    return int(lib().orc_fp8_code(float(x), float(scale)))


def fp8_quantize_to_pool(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, num_pages: int,
                         k_scale: float = 1.0, v_scale: float = 1.0, pool: np.ndarray | None = None) -> np.ndarray:
    """k, v: [T, Hkv, 128] float32 or uint16 (bf16 bits). Returns the FP8 pool."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    assert k.shape == v.shape and k.dtype == v.dtype and k.shape[2] == HEAD_DIM
    T, hkv, _ = k.shape
    dtype = 0 if k.dtype == np.float32 else 1
    assert dtype == 0 or k.dtype == np.uint16
    if pool is None:
        pool = np.zeros(fp8_pool_bytes(num_pages, hkv), dtype=np.uint8)
    sm = np.ascontiguousarray(slot_mapping.astype(np.int32, copy=False))
    lib().orc_fp8_quantize_to_pool(_ptr(k), _ptr(v), dtype, hkv * HEAD_DIM, HEAD_DIM, _ptr(sm), T, hkv,
                                   float(k_scale), float(v_scale), _ptr(pool))
    return pool


def fp8_dequant_row(pool: np.ndarray, page: int, row: int, head: int, kind: int, num_kv_heads: int,
                    scale: float = 1.0) -> np.ndarray:
    out = np.zeros(HEAD_DIM, dtype=np.float64)
    lib().orc_fp8_dequant_row(_ptr(pool), int(page), int(row), int(head), int(kind), int(num_kv_heads),
                              float(scale), _ptr(out))
    return out


def fp8_decode_attn(q_bf16_bits: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray, pool: np.ndarray,
                    num_kv_heads: int, sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0, units=None,
                    n_threads: int = 1):
    """Decode attention over the FP8 baseline pool; same conventions as decode_attn."""
    q = np.ascontiguousarray(q_bf16_bits.astype(np.uint16, copy=False))
    B, hq, d = q.shape
    assert d == HEAD_DIM and hq % num_kv_heads == 0
    pt = np.ascontiguousarray(page_table.astype(np.int32, copy=False))
    sl = np.ascontiguousarray(seq_lens.astype(np.int32, copy=False))
    out = np.full((B, hq, HEAD_DIM), np.nan, dtype=np.float64)
    lse = np.full((B, hq), np.nan, dtype=np.float64)
    if units is None:
        u_ptr, n_u = None, B * hq
    else:
        u_arr = np.ascontiguousarray(np.asarray(list(units), dtype=np.int32))
        u_ptr, n_u = _ptr(u_arr), len(u_arr)
    lib().orc_fp8_decode_attn(_ptr(q), _ptr(pt), pt.shape[1], _ptr(sl), B, hq, num_kv_heads, _ptr(pool),
                              float(k_scale), float(v_scale), float(sm_scale), _ptr(out), _ptr(lse), u_ptr, n_u,
                              int(n_threads))
    return out, lse


# ---- global-scale calibration -------------------------------------------------
def amax(x: np.ndarray) -> float:
    """max |x| of a [T, H, 128] float32 or uint16 (bf16 bits) array."""
    x = np.ascontiguousarray(x)
    T, H, d = x.shape
    assert d == HEAD_DIM and x.dtype in (np.float32, np.uint16)
    return float(lib().orc_amax(_ptr(x), 0 if x.dtype == np.float32 else 1, H * HEAD_DIM, HEAD_DIM, T, H))


def global_scale_for_amax(a: float) -> float:
    return float(lib().orc_global_scale_for_amax(float(a)))


def global_scale_tight_for_amax(a: float) -> float:
    """Smallest binary32 g with a / (6 g) <= 448 (1.0 for a = 0)."""
    return float(lib().orc_global_scale_tight_for_amax(float(a)))


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of the bf16 values nearest to the float64 values x,
    ties to even: one rounding of exact values (e.g. a dequantized workspace)."""
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.zeros(xa.shape, dtype=np.uint16)
    lib().orc_bf16_bits_of_array(_ptr(xa), xa.size, _ptr(out))
    return out
