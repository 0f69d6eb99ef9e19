"""Thin ctypes binding of libnvfp4kv (include/nvfp4kv.h).

Argument marshalling only: every step of the path runs in the HIP kernels of the
library. PyTorch supplies device memory and streams. Every function raises
RuntimeError when the library returns a non-zero status, and importing the
library fails loudly when it has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4kv.so")

HEAD_DIM = 128
PAGE_SIZE = 16
SLAB_BYTES = 1152
F32 = 0
BF16 = 1
FP8_E4M3 = 2  # extend workspace only
F16_TILED = 3  # extend workspace: K bf16 rows, V f16 tiles of 64 rows

EXPORTED = [
    "nvfp4kv_pool_bytes",
    "nvfp4kv_status_string",
    "nvfp4kv_version",
    "nvfp4_kv_quantize",
    "nvfp4_paged_decode_attn_default_splits",
    "nvfp4_paged_decode_attn_workspace_bytes",
    "nvfp4_paged_decode_attn",
    "nvfp4_paged_decode_attn_partial",
    "nvfp4_decode_combine",
    "nvfp4_paged_decode_attn_append",
    "nvfp4_kv_dequant_workspace",
    "nvfp4_extend_attn",
    "nvfp4_kv_amax_workspace_bytes",
    "nvfp4_kv_amax",
    "nvfp4kv_global_scale_for_amax",
    "nvfp4kv_global_scale_tight_for_amax",
    "fp8kv_pool_bytes",
    "fp8_kv_quantize",
    "fp8_paged_decode_attn_default_splits",
    "fp8_paged_decode_attn",
    "fp8_paged_decode_attn_partial",
    "fp8_paged_decode_attn_append",
    "nvfp4_paged_decode_attn_noalloc",
    "nvfp4kv_check_page_table",
    "nvfp4kv_tiled_v_bytes",
]


class PoolDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("num_kv_heads", ctypes.c_int32),
                ("global_scale", ctypes.c_float)]


class Fp8PoolDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("num_kv_heads", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m bit_paged_kv_nvfp4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        P = c.c_void_p
        L.nvfp4kv_pool_bytes.argtypes = [c.c_int64, c.c_int32]
        L.nvfp4kv_pool_bytes.restype = c.c_int64
        L.nvfp4kv_status_string.argtypes = [c.c_int32]
        L.nvfp4kv_status_string.restype = c.c_char_p
        L.nvfp4kv_version.argtypes = []
        L.nvfp4kv_version.restype = c.c_int32
        L.nvfp4_kv_quantize.argtypes = [P, P, c.c_int32, c.c_int64, c.c_int64, P, c.c_int64,
                                        c.POINTER(PoolDesc), P]
        L.nvfp4_kv_quantize.restype = c.c_int32
        L.nvfp4_paged_decode_attn_default_splits.argtypes = [c.c_int32, c.c_int32, c.c_int32, c.c_int32]
        L.nvfp4_paged_decode_attn_default_splits.restype = c.c_int32
        L.nvfp4_paged_decode_attn_workspace_bytes.argtypes = [c.c_int32, c.c_int32, c.c_int32]
        L.nvfp4_paged_decode_attn_workspace_bytes.restype = c.c_size_t
        L.nvfp4_paged_decode_attn.argtypes = [P, P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int32,
                                              c.POINTER(PoolDesc), c.c_float, c.c_int32, P, c.c_size_t, P,
                                              c.c_int32, P, P]
        L.nvfp4_paged_decode_attn.restype = c.c_int32
        L.nvfp4_paged_decode_attn_partial.argtypes = [P, P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int32,
                                                      c.POINTER(PoolDesc), c.c_float, c.c_int32, P, c.c_size_t, P]
        L.nvfp4_paged_decode_attn_partial.restype = c.c_int32
        append_args = [P, P, P, c.c_int32, c.c_int64, c.c_int64, P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int32]
        tail_args = [c.c_float, c.c_int32, P, c.c_size_t, P, c.c_int32, P, P]
        L.nvfp4_paged_decode_attn_append.argtypes = append_args + [c.POINTER(PoolDesc)] + tail_args
        L.nvfp4_paged_decode_attn_append.restype = c.c_int32
        L.fp8_paged_decode_attn_append.argtypes = append_args + [c.POINTER(Fp8PoolDesc)] + tail_args
        L.fp8_paged_decode_attn_append.restype = c.c_int32
        L.nvfp4_decode_combine.argtypes = [P, c.c_size_t, c.c_int32, c.c_int32, c.c_int32, P, c.c_int32, P, P]
        L.nvfp4_decode_combine.restype = c.c_int32
        L.nvfp4_kv_dequant_workspace.argtypes = [c.POINTER(PoolDesc), P, c.c_int64, P, P, c.c_int32, c.c_int32,
                                                 P, P, c.c_int32, P]
        L.nvfp4_kv_dequant_workspace.restype = c.c_int32
        L.nvfp4_extend_attn.argtypes = [P, P, P, c.c_int32, c.c_int64, P, P, c.c_int64, c.c_int32, c.c_int32,
                                        c.c_float, c.c_float, P, P, c.POINTER(PoolDesc), P, P]
        L.nvfp4_extend_attn.restype = c.c_int32
        L.nvfp4_kv_amax_workspace_bytes.argtypes = []
        L.nvfp4_kv_amax_workspace_bytes.restype = c.c_size_t
        L.nvfp4_kv_amax.argtypes = [P, P, c.c_int32, c.c_int64, c.c_int64, c.c_int64, c.c_int32, P, P, c.c_size_t, P]
        L.nvfp4_kv_amax.restype = c.c_int32
        L.nvfp4kv_global_scale_for_amax.argtypes = [c.c_float]
        L.nvfp4kv_global_scale_for_amax.restype = c.c_float
        L.nvfp4kv_global_scale_tight_for_amax.argtypes = [c.c_float]
        L.nvfp4kv_global_scale_tight_for_amax.restype = c.c_float
        L.fp8kv_pool_bytes.argtypes = [c.c_int64, c.c_int32]
        L.fp8kv_pool_bytes.restype = c.c_int64
        L.fp8_kv_quantize.argtypes = [P, P, c.c_int32, c.c_int64, c.c_int64, P, c.c_int64, c.POINTER(Fp8PoolDesc), P]
        L.fp8_kv_quantize.restype = c.c_int32
        L.fp8_paged_decode_attn_default_splits.argtypes = [c.c_int32, c.c_int32, c.c_int32, c.c_int32]
        L.fp8_paged_decode_attn_default_splits.restype = c.c_int32
        L.fp8_paged_decode_attn.argtypes = [P, P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int32,
                                            c.POINTER(Fp8PoolDesc), c.c_float, c.c_int32, P, c.c_size_t, P,
                                            c.c_int32, P, P]
        L.fp8_paged_decode_attn.restype = c.c_int32
        L.fp8_paged_decode_attn_partial.argtypes = [P, P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int32,
                                                    c.POINTER(Fp8PoolDesc), c.c_float, c.c_int32, P, c.c_size_t, P]
        L.fp8_paged_decode_attn_partial.restype = c.c_int32
        L.nvfp4_paged_decode_attn_noalloc.argtypes = [P, P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int32,
                                                      c.POINTER(PoolDesc), c.c_float, c.c_int32, P, c.c_int32, P, P]
        L.nvfp4_paged_decode_attn_noalloc.restype = c.c_int32
        L.nvfp4kv_check_page_table.argtypes = [P, c.c_int64, P, c.c_int32, c.c_int32, c.c_int64, P,
                                               c.POINTER(c.c_int64)]
        L.nvfp4kv_check_page_table.restype = c.c_int32
        L.nvfp4kv_tiled_v_bytes.argtypes = [c.c_int64, c.c_int32]
        L.nvfp4kv_tiled_v_bytes.restype = c.c_int64
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().nvfp4kv_status_string(int(code)).decode()


def _check(name: str, code: int) -> None:
    if code != 0:
        raise RuntimeError(f"{name} failed with status {code}: {status_string(code)}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _same_device(ref: torch.Tensor, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, q on {ref.device}: every tensor must be on one device")


def _decode_inputs(q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, pool, max_seq_len: int):
    """Checks the decode inputs against the header's contract and returns (B, Hq).
    The kernels read seq_lens as int32 [B] and q as bf16 [B, Hq, 128]; a tensor of
    another dtype or size would be read as wrong values or past its end."""
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [B, Hq, 128] tensor")
    B, hq, _ = q.shape
    if hq % pool.num_kv_heads != 0:
        raise ValueError(f"num_q_heads {hq} is not a multiple of the pool's {pool.num_kv_heads} KV heads")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous():
        raise ValueError("page_table must be contiguous int32 [B, stride]")
    if page_table.shape[0] < B:
        raise ValueError(f"page_table has {page_table.shape[0]} rows for a batch of {B}")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError(f"seq_lens must be a contiguous int32 tensor of {B} entries (got {seq_lens.dtype} "
                         f"{tuple(seq_lens.shape)})")
    if int(max_seq_len) > page_table.shape[1] * PAGE_SIZE:
        raise ValueError(f"max_seq_len {max_seq_len} exceeds the page table row ({page_table.shape[1]} pages)")
    _same_device(q, page_table=page_table, seq_lens=seq_lens, pool=pool.data)
    return B, hq


def _outputs(q: torch.Tensor, B: int, hq: int, out: torch.Tensor | None, out_dtype, lse: torch.Tensor | None):
    """The combine writes out [B, Hq, 128] (f32 or bf16) and lse f32 [B, Hq]: any
    other shape would be written past its end. Returns (out, dtype code)."""
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=out_dtype, device=q.device)
    odt = {torch.float32: F32, torch.bfloat16: BF16}.get(out.dtype)
    if odt is None or not out.is_contiguous() or tuple(out.shape) != (B, hq, HEAD_DIM):
        raise ValueError(f"out must be a contiguous float32 or bfloat16 [{B}, {hq}, 128] tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, hq)):
        raise ValueError(f"lse must be a contiguous float32 [{B}, {hq}] tensor")
    _same_device(q, out=out, lse=lse)
    return out, odt


def _workspace(q: torch.Tensor, workspace: torch.Tensor | None, B: int, hq: int, num_splits: int) -> torch.Tensor:
    nbytes = nvfp4_paged_decode_attn_workspace_bytes(B, hq, num_splits)
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _same_device(q, workspace=workspace)
    return workspace


class Pool:
    """NVFP4 KV pool of one layer: a device uint8 buffer of num_pages pages with
    num_kv_heads K and V slabs each (layout in include/nvfp4kv.h)."""

    def __init__(self, num_pages: int, num_kv_heads: int, device="cuda", global_scale: float = 1.0,
                 data: torch.Tensor | None = None):
        nbytes = nvfp4kv_pool_bytes(num_pages, num_kv_heads)
        if data is None:
            data = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        if data.numel() != nbytes or data.dtype != torch.uint8:
            raise ValueError("pool buffer has the wrong size or dtype")
        self.data = data
        self.num_pages = int(num_pages)
        self.num_kv_heads = int(num_kv_heads)
        self.global_scale = float(global_scale)

    def desc(self) -> PoolDesc:
        return PoolDesc(self.data.data_ptr(), self.num_pages, self.num_kv_heads, self.global_scale)


class Fp8Pool:
    """FP8 E4M3 baseline pool of one layer (layout in include/nvfp4kv.h)."""

    def __init__(self, num_pages: int, num_kv_heads: int, device="cuda", k_scale: float = 1.0,
                 v_scale: float = 1.0, data: torch.Tensor | None = None):
        nbytes = fp8kv_pool_bytes(num_pages, num_kv_heads)
        if data is None:
            data = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        if data.numel() != nbytes or data.dtype != torch.uint8:
            raise ValueError("pool buffer has the wrong size or dtype")
        self.data = data
        self.num_pages = int(num_pages)
        self.num_kv_heads = int(num_kv_heads)
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)

    def desc(self) -> Fp8PoolDesc:
        return Fp8PoolDesc(self.data.data_ptr(), self.num_pages, self.num_kv_heads, self.k_scale, self.v_scale)


def fp8kv_pool_bytes(num_pages: int, num_kv_heads: int) -> int:
    return int(lib().fp8kv_pool_bytes(int(num_pages), int(num_kv_heads)))


def nvfp4kv_pool_bytes(num_pages: int, num_kv_heads: int) -> int:
    return int(lib().nvfp4kv_pool_bytes(int(num_pages), int(num_kv_heads)))


def _quantize(name, k, v, slot_mapping, pool, stream):
    if k.dtype != v.dtype or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share dtype, shape and strides")
    if k.dim() != 3 or k.shape[2] != HEAD_DIM or k.stride(2) != 1:
        raise ValueError("k, v must be [T, Hkv, 128] with a contiguous last dimension")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(k.dtype)
    if dt is None:
        raise ValueError("k, v must be float32 or bfloat16")
    if slot_mapping.dtype != torch.int32 or slot_mapping.numel() != k.shape[0]:
        raise ValueError("slot_mapping must be int32 [T]")
    d = pool.desc()
    _check(name, getattr(lib(), name)(_ptr(k), _ptr(v), dt, k.stride(0), k.stride(1), _ptr(slot_mapping), k.shape[0],
                                      ctypes.byref(d), _stream(stream)))


def fp8_kv_quantize(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, pool: Fp8Pool, stream=None):
    """As nvfp4_kv_quantize, into an FP8 baseline pool."""
    _quantize("fp8_kv_quantize", k, v, slot_mapping, pool, stream)


def nvfp4_kv_quantize(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, pool: Pool, stream=None):
    """k, v: [T, Hkv, 128] float32 or bfloat16 on the device (last dim contiguous);
    slot_mapping: int32 [T] (negative = skip)."""
    _quantize("nvfp4_kv_quantize", k, v, slot_mapping, pool, stream)


def nvfp4_paged_decode_attn_default_splits(batch: int, num_kv_heads: int, max_seq_len: int, num_cus: int = 0) -> int:
    return int(lib().nvfp4_paged_decode_attn_default_splits(batch, num_kv_heads, max_seq_len, num_cus))


def nvfp4_paged_decode_attn_workspace_bytes(batch: int, num_q_heads: int, num_splits: int) -> int:
    return int(lib().nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, num_splits))


def nvfp4_paged_decode_attn(q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Pool,
                            sm_scale: float, max_seq_len: int, num_splits: int = 0,
                            workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                            out_dtype: torch.dtype = torch.bfloat16, lse: torch.Tensor | None = None, stream=None):
    """q: bf16 [B, Hq, 128]; page_table: int32 [>= B, stride]; seq_lens: int32 [B].
    Returns out [B, Hq, 128] (and fills ``lse`` [B, Hq] float32 when given)."""
    B, hq = _decode_inputs(q, page_table, seq_lens, pool, max_seq_len)
    if num_splits == 0:
        num_splits = nvfp4_paged_decode_attn_default_splits(B, pool.num_kv_heads, max_seq_len)
    workspace = _workspace(q, workspace, B, hq, num_splits)
    out, odt = _outputs(q, B, hq, out, out_dtype, lse)
    d = pool.desc()
    _check("nvfp4_paged_decode_attn",
           lib().nvfp4_paged_decode_attn(_ptr(q), _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, hq,
                                         int(max_seq_len), ctypes.byref(d), float(sm_scale), int(num_splits),
                                         _ptr(workspace), workspace.numel(), _ptr(out), odt, _ptr(lse),
                                         _stream(stream)))
    return out


def nvfp4_paged_decode_attn_noalloc(q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Pool,
                                    sm_scale: float, max_seq_len: int, num_splits: int = 0, out: torch.Tensor | None = None,
                                    out_dtype: torch.dtype = torch.bfloat16, lse: torch.Tensor | None = None,
                                    stream=None):
    """As nvfp4_paged_decode_attn, with the split states in the library's fixed
    per-GPU scratch array instead of a workspace (no device allocation by the
    library; ``out`` is allocated here only when not given)."""
    B, hq = _decode_inputs(q, page_table, seq_lens, pool, max_seq_len)
    out, odt = _outputs(q, B, hq, out, out_dtype, lse)
    d = pool.desc()
    _check("nvfp4_paged_decode_attn_noalloc",
           lib().nvfp4_paged_decode_attn_noalloc(_ptr(q), _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, hq,
                                                 int(max_seq_len), ctypes.byref(d), float(sm_scale), int(num_splits),
                                                 _ptr(out), odt, _ptr(lse), _stream(stream)))
    return out


def _decode_append(name: str, default_splits, q, k_new, v_new, page_table, seq_lens, pool, sm_scale, max_seq_len,
                   num_splits, workspace, out, out_dtype, lse, stream, combine):
    B, hq = _decode_inputs(q, page_table, seq_lens, pool, max_seq_len)
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 3 or tuple(t.shape) != (B, pool.num_kv_heads, HEAD_DIM) or t.stride(2) != 1:
            raise ValueError(f"{nm} must be [B, Hkv, 128] with unit channel stride")
    if k_new.dtype != v_new.dtype or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share dtype and strides")
    ndt = {torch.float32: F32, torch.bfloat16: BF16}.get(k_new.dtype)
    if ndt is None:
        raise ValueError("k_new/v_new must be float32 or bfloat16")
    _same_device(q, k_new=k_new, v_new=v_new)
    if num_splits == 0:
        num_splits = default_splits(B, pool.num_kv_heads, max_seq_len)
    if not combine:
        if workspace is None or out is not None or lse is not None:
            raise ValueError("phase 1 alone needs a workspace and takes no out/lse")
        odt = F32
    else:
        out, odt = _outputs(q, B, hq, out, out_dtype, lse)
    workspace = _workspace(q, workspace, B, hq, num_splits)
    d = pool.desc()
    _check(name, getattr(lib(), name)(_ptr(q), _ptr(k_new), _ptr(v_new), ndt, k_new.stride(0), k_new.stride(1),
                                      _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, hq, int(max_seq_len),
                                      ctypes.byref(d), float(sm_scale), int(num_splits), _ptr(workspace),
                                      workspace.numel(), _ptr(out), odt, _ptr(lse), _stream(stream)))
    return out


def nvfp4_paged_decode_attn_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                   page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Pool, sm_scale: float,
                                   max_seq_len: int, num_splits: int = 0, workspace: torch.Tensor | None = None,
                                   out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                                   lse: torch.Tensor | None = None, stream=None, combine: bool = True):
    """One decode step in one split launch: writes k_new/v_new [B, Hkv, 128]
    (float32 or bfloat16) as token seq_lens[b] - 1 of each sequence into the pool,
    then attends as nvfp4_paged_decode_attn over the updated cache. With
    combine=False only phase 1 runs (states left in ``workspace``; returns None)."""
    return _decode_append("nvfp4_paged_decode_attn_append", nvfp4_paged_decode_attn_default_splits, q, k_new, v_new,
                          page_table, seq_lens, pool, sm_scale, max_seq_len, num_splits, workspace, out, out_dtype,
                          lse, stream, combine)


def nvfp4_paged_decode_attn_partial(q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Pool,
                                    sm_scale: float, max_seq_len: int, num_splits: int, workspace: torch.Tensor,
                                    stream=None):
    """Phase 1: per-split online-softmax states into ``workspace`` (layout in the C header)."""
    B, hq = _decode_inputs(q, page_table, seq_lens, pool, max_seq_len)
    workspace = _workspace(q, workspace, B, hq, int(num_splits))
    d = pool.desc()
    _check("nvfp4_paged_decode_attn_partial",
           lib().nvfp4_paged_decode_attn_partial(_ptr(q), _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, hq,
                                                 int(max_seq_len), ctypes.byref(d), float(sm_scale), int(num_splits),
                                                 _ptr(workspace), workspace.numel(), _stream(stream)))


def nvfp4_decode_combine(workspace: torch.Tensor, batch: int, num_q_heads: int, num_splits: int, out: torch.Tensor,
                         lse: torch.Tensor | None = None, stream=None):
    """Phase 2: merge the split states into ``out`` (float32 or bfloat16 [B, Hq, 128])."""
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    out, odt = _outputs(workspace, int(batch), int(num_q_heads), out, None, lse)
    _check("nvfp4_decode_combine",
           lib().nvfp4_decode_combine(_ptr(workspace), workspace.numel(), int(batch), int(num_q_heads), int(num_splits),
                                      _ptr(out), odt, _ptr(lse), _stream(stream)))
    return out


def nvfp4_kv_dequant_workspace(pool: Pool, page_table: torch.Tensor, seq_lens: torch.Tensor,
                               row_offsets: torch.Tensor, max_seq_len: int, k_out: torch.Tensor,
                               v_out: torch.Tensor, stream=None):
    """Writes K^, V^ rows [row_offsets[s] + t] of k_out / v_out ([rows, Hkv, 128],
    float32, bfloat16 or float8_e4m3fn) for t < seq_lens[s]."""
    n = seq_lens.numel()
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [n_seqs] tensor")
    if row_offsets.dtype != torch.int64 or tuple(row_offsets.shape) != (n,) or not row_offsets.is_contiguous():
        raise ValueError(f"row_offsets must be a contiguous int64 tensor of {n} entries")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous() or \
            page_table.shape[0] < n:
        raise ValueError(f"page_table must be contiguous int32 [>= {n}, stride]")
    if int(max_seq_len) > page_table.shape[1] * PAGE_SIZE:
        raise ValueError(f"max_seq_len {max_seq_len} exceeds the page table row ({page_table.shape[1]} pages)")
    if not k_out.is_contiguous() or not v_out.is_contiguous():
        raise ValueError("k_out and v_out must be contiguous")
    if k_out.dim() != 3 or k_out.shape[1:] != (pool.num_kv_heads, HEAD_DIM):
        raise ValueError(f"k_out must be [rows, {pool.num_kv_heads}, 128]")
    tiled = k_out.dtype == torch.bfloat16 and v_out.dtype == torch.float16
    if tiled:
        if v_out.dim() != 4 or v_out.shape[1:] != (pool.num_kv_heads, HEAD_DIM, 64) or \
                v_out.shape[0] * 64 < k_out.shape[0]:
            raise ValueError(f"a tiled v_out must be float16 [>= rows / 64, {pool.num_kv_heads}, 128, 64]")
    elif k_out.dtype != v_out.dtype or k_out.shape != v_out.shape:
        raise ValueError(f"k_out and v_out must share dtype and shape [rows, {pool.num_kv_heads}, 128] "
                         "(or be bfloat16 rows and float16 tiles)")
    _same_device(k_out, v_out=v_out, page_table=page_table, seq_lens=seq_lens, row_offsets=row_offsets,
                 pool=pool.data)
    odt = F16_TILED if tiled else {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}.get(k_out.dtype)
    if odt is None:
        raise ValueError("workspace dtype must be float32, bfloat16 or float8_e4m3fn")
    d = pool.desc()
    _check("nvfp4_kv_dequant_workspace",
           lib().nvfp4_kv_dequant_workspace(ctypes.byref(d), _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                                            _ptr(row_offsets), seq_lens.numel(), int(max_seq_len), _ptr(k_out),
                                            _ptr(v_out), odt, _stream(stream)))


def nvfp4_extend_attn(q: torch.Tensor, k_prefix: torch.Tensor, v_prefix: torch.Tensor, k_chunk: torch.Tensor,
                      v_chunk: torch.Tensor, sm_scale: float, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, chunk_pool: "Pool | None" = None,
                      chunk_slots: torch.Tensor | None = None, v_bound: float = 0.0, stream=None) -> torch.Tensor:
    """Chunk queries q [C, Hq, 128] (bf16) over the prefix workspace k/v_prefix
    [P, Hkv, 128] (bfloat16 or float8_e4m3fn) and the chunk's own k/v_chunk
    [C, Hkv, 128] (bf16), causal over the chunk. Returns out [C, Hq, 128] bf16;
    fills lse [C, Hq] (float32, natural log) when given. With chunk_pool and
    chunk_slots (int32 [C]) the same launch quantize-writes the chunk into the pool.
    ``v_bound``: an upper bound of |V| over the workspace and the chunk (0 when it
    is below 2^15; a workspace dequantized at global scale g is bounded by 2688 g)."""
    if (chunk_pool is None) != (chunk_slots is None):
        raise ValueError("chunk_pool and chunk_slots go together")
    if chunk_slots is not None and (chunk_slots.dtype != torch.int32 or chunk_slots.numel() != q.shape[0]):
        raise ValueError("chunk_slots must be int32 [C]")
    for name, t in (("q", q), ("k_chunk", k_chunk), ("v_chunk", v_chunk)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous bfloat16")
    if not k_prefix.is_contiguous() or not v_prefix.is_contiguous():
        raise ValueError("k_prefix and v_prefix must be contiguous")
    tiled = k_prefix.dtype == torch.bfloat16 and v_prefix.dtype == torch.float16
    if not tiled and k_prefix.dtype != v_prefix.dtype:
        raise ValueError("k_prefix and v_prefix must share a dtype (or be bfloat16 rows and float16 tiles)")
    pdt = F16_TILED if tiled else {torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}.get(k_prefix.dtype)
    if pdt is None:
        raise ValueError("prefix workspace dtype must be bfloat16 or float8_e4m3fn")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or k_prefix.dim() != 3 or k_chunk.dim() != 3:
        raise ValueError("q, k/v_prefix and k/v_chunk must be [rows, heads, 128]")
    C, hq, _ = q.shape
    P, hkv, _ = k_prefix.shape
    if tuple(k_prefix.shape) != (P, hkv, HEAD_DIM):
        raise ValueError("k_prefix must be [P, Hkv, 128]")
    if tiled:
        if v_prefix.dim() != 4 or v_prefix.shape[1:] != (hkv, HEAD_DIM, 64) or v_prefix.shape[0] * 64 < P:
            raise ValueError("a tiled v_prefix must be float16 [>= P / 64, Hkv, 128, 64]")
    elif v_prefix.shape != k_prefix.shape:
        raise ValueError("k_prefix and v_prefix must both be [P, Hkv, 128]")
    if tuple(k_chunk.shape) != (C, hkv, HEAD_DIM) or v_chunk.shape != k_chunk.shape:
        raise ValueError(f"k_chunk and v_chunk must both be [{C}, {hkv}, 128]")
    if out is None:
        out = torch.empty_like(q)
    if out.dtype != torch.bfloat16 or not out.is_contiguous() or out.shape != q.shape:
        raise ValueError(f"out must be a contiguous bfloat16 [{C}, {hq}, 128] tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (C, hq)):
        raise ValueError(f"lse must be a contiguous float32 [{C}, {hq}] tensor")
    _same_device(q, k_prefix=k_prefix, v_prefix=v_prefix, k_chunk=k_chunk, v_chunk=v_chunk, out=out, lse=lse,
                 chunk_slots=chunk_slots)
    _check("nvfp4_extend_attn",
           lib().nvfp4_extend_attn(_ptr(q), _ptr(k_prefix) if P else None, _ptr(v_prefix) if P else None, pdt, P,
                                   _ptr(k_chunk), _ptr(v_chunk), C, hq, hkv, float(sm_scale), float(v_bound),
                                   _ptr(out), _ptr(lse),
                                   ctypes.byref(chunk_pool.desc()) if chunk_pool is not None else None,
                                   _ptr(chunk_slots), _stream(stream)))
    return out


def fp8_paged_decode_attn_default_splits(batch: int, num_kv_heads: int, max_seq_len: int, num_cus: int = 0) -> int:
    return int(lib().fp8_paged_decode_attn_default_splits(batch, num_kv_heads, max_seq_len, num_cus))


def fp8_paged_decode_attn(q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Fp8Pool,
                          sm_scale: float, max_seq_len: int, num_splits: int = 0,
                          workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                          out_dtype: torch.dtype = torch.bfloat16, lse: torch.Tensor | None = None, stream=None):
    """As nvfp4_paged_decode_attn, over an FP8 baseline pool."""
    B, hq = _decode_inputs(q, page_table, seq_lens, pool, max_seq_len)
    if num_splits == 0:
        num_splits = fp8_paged_decode_attn_default_splits(B, pool.num_kv_heads, max_seq_len)
    workspace = _workspace(q, workspace, B, hq, num_splits)
    out, odt = _outputs(q, B, hq, out, out_dtype, lse)
    d = pool.desc()
    _check("fp8_paged_decode_attn",
           lib().fp8_paged_decode_attn(_ptr(q), _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, hq,
                                       int(max_seq_len), ctypes.byref(d), float(sm_scale), int(num_splits),
                                       _ptr(workspace), workspace.numel(), _ptr(out), odt, _ptr(lse),
                                       _stream(stream)))
    return out


def fp8_paged_decode_attn_partial(q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Fp8Pool,
                                  sm_scale: float, max_seq_len: int, num_splits: int, workspace: torch.Tensor,
                                  stream=None):
    """Phase 1 over an FP8 baseline pool (phase 2 is nvfp4_decode_combine)."""
    B, hq = _decode_inputs(q, page_table, seq_lens, pool, max_seq_len)
    workspace = _workspace(q, workspace, B, hq, int(num_splits))
    d = pool.desc()
    _check("fp8_paged_decode_attn_partial",
           lib().fp8_paged_decode_attn_partial(_ptr(q), _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B,
                                               hq, int(max_seq_len), ctypes.byref(d), float(sm_scale),
                                               int(num_splits), _ptr(workspace), workspace.numel(), _stream(stream)))


def fp8_paged_decode_attn_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                 page_table: torch.Tensor, seq_lens: torch.Tensor, pool: Fp8Pool, sm_scale: float,
                                 max_seq_len: int, num_splits: int = 0, workspace: torch.Tensor | None = None,
                                 out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                                 lse: torch.Tensor | None = None, stream=None, combine: bool = True):
    """As nvfp4_paged_decode_attn_append, over an FP8 baseline pool."""
    return _decode_append("fp8_paged_decode_attn_append", fp8_paged_decode_attn_default_splits, q, k_new, v_new,
                          page_table, seq_lens, pool, sm_scale, max_seq_len, num_splits, workspace, out, out_dtype,
                          lse, stream, combine)


def nvfp4_kv_amax(k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """max |K| and max |V| of [T, Hkv, 128] float32/bfloat16 tensors, as a device
    float32 [2] tensor (NaN elements ignored)."""
    if k.dtype != v.dtype or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share dtype, shape and strides")
    if k.dim() != 3 or k.shape[2] != HEAD_DIM or k.stride(2) != 1:
        raise ValueError("k, v must be [T, Hkv, 128] with a contiguous last dimension")
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(k.dtype)
    if dt is None:
        raise ValueError("k, v must be float32 or bfloat16")
    if out is None:
        out = torch.empty(2, dtype=torch.float32, device=k.device)
    ws = torch.empty(int(lib().nvfp4_kv_amax_workspace_bytes()), dtype=torch.uint8, device=k.device)
    _check("nvfp4_kv_amax", lib().nvfp4_kv_amax(_ptr(k), _ptr(v), dt, k.stride(0), k.stride(1), k.shape[0], k.shape[1],
                                                _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def nvfp4kv_global_scale_for_amax(amax: float) -> float:
    return float(lib().nvfp4kv_global_scale_for_amax(float(amax)))


def nvfp4kv_global_scale_tight_for_amax(amax: float) -> float:
    return float(lib().nvfp4kv_global_scale_tight_for_amax(float(amax)))


def nvfp4kv_check_page_table(page_table, seq_lens, max_seq_len: int, num_pages: int, exclusive: bool = False) -> None:
    """CPU check of the decode inputs' data preconditions (page ids inside the
    pool, lengths within max_seq_len and the table row; with ``exclusive``, no
    physical page holding live tokens of two sequences). Takes host arrays (numpy,
    or CPU tensors) and raises ValueError naming the first offending entry."""
    import numpy as np

    pt = np.ascontiguousarray(np.asarray(page_table), dtype=np.int32)
    sl = np.ascontiguousarray(np.asarray(seq_lens), dtype=np.int32)
    if pt.ndim != 2 or sl.ndim != 1 or pt.shape[0] < sl.shape[0]:
        raise ValueError("page_table must be [>= B, stride] and seq_lens [B]")
    seen = np.zeros(int(num_pages), dtype=np.uint8) if exclusive else None
    bad = ctypes.c_int64(-1)
    code = lib().nvfp4kv_check_page_table(pt.ctypes.data, pt.shape[1], sl.ctypes.data, sl.shape[0],
                                          int(max_seq_len), int(num_pages),
                                          None if seen is None else seen.ctypes.data, ctypes.byref(bad))
    if code == 2 and bad.value >= 0:
        raise ValueError(f"seq_lens[{bad.value}] = {int(sl[bad.value])} is negative or exceeds max_seq_len "
                         f"{max_seq_len} or the page table row ({pt.shape[1]} pages)")
    if code == 6:
        b, p = divmod(bad.value, pt.shape[1])
        raise ValueError(f"page_table[{b}][{p}] = {int(pt[b, p])} is outside the pool of {num_pages} pages"
                         + (" or already holds live tokens" if exclusive else ""))
    _check("nvfp4kv_check_page_table", code)


def nvfp4kv_tiled_v_bytes(rows: int, num_kv_heads: int) -> int:
    return int(lib().nvfp4kv_tiled_v_bytes(int(rows), int(num_kv_heads)))


def tiled_v_workspace(rows: int, num_kv_heads: int, device="cuda") -> torch.Tensor:
    """A float16 [ceil(rows / 64), Hkv, 128, 64] tensor for the V part of an
    NVFP4KV_F16_TILED workspace (layout in the C header)."""
    return torch.empty(((rows + 63) // 64, num_kv_heads, HEAD_DIM, 64), dtype=torch.float16, device=device)
