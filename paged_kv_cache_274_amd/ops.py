"""Thin ctypes binding of libpkv.so (include/pkv.h), same call names.

Argument marshalling only: shapes and dtypes are checked, torch tensors are
passed as device pointers together with torch's current HIP stream, and every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if ``libpkv.so`` is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_BF16, PKV_INT8 = 0, 1, 2
_DTYPE = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}
_WS_DTYPE = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.int8: PKV_INT8}
EXPORTED = ("kv_append", "paged_decode_attention", "paged_prefill_attention",
            "kv_append_int8", "paged_decode_attention_int8",
            "pkv_decode_workspace_bytes", "pkv_decode_num_splits", "pkv_status_string",
            "paged_decode_attention_split", "pkv_decode_workspace_bytes_split",
            "paged_decode_attention_noalloc", "paged_prefill_attention_int8",
            "copy_blocks", "swap_blocks",
            "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add_sequence", "pkv_bm_append",
            "pkv_bm_fork", "pkv_bm_free", "pkv_bm_swap_out", "pkv_bm_swap_in",
            "pkv_bm_block_table", "pkv_bm_get_stats", "pkv_kv_cache_bytes",
            "pkv_bm_append_batch", "pkv_bm_block_tables",
            "pkv_decode_line_start", "pkv_decode_line_wave_of")
PKV_ERR_NO_BLOCKS = 5

_lib = None


class PkvError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what} failed: {status_string(status)} ({status})")
        self.status = status


class NoBlocksError(PkvError):
    """The block manager has too few free blocks; nothing changed."""


class BlockManagerStats(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("cached_blocks", ctypes.c_int32), ("cached_free_blocks", ctypes.c_int32),
                ("n_host_blocks", ctypes.c_int32), ("host_free_blocks", ctypes.c_int32),
                ("n_sequences", ctypes.c_int32), ("hit_tokens", ctypes.c_int64),
                ("query_tokens", ctypes.c_int64), ("hit_requests", ctypes.c_int64),
                ("requests", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """Load libpkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m paged_kv_cache_274_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p, i32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    L.pkv_status_string.argtypes = [i32]
    L.pkv_status_string.restype = ctypes.c_char_p
    L.kv_append.argtypes = [vp, vp, i64p, vp, vp, i32, i32, i32, i32, i32, vp]
    L.kv_append.restype = i32
    L.pkv_decode_num_splits.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pkv_decode_num_splits.restype = i32
    L.pkv_decode_line_start.argtypes = [ctypes.c_int64, i32, i32]
    L.pkv_decode_line_start.restype = ctypes.c_int64
    L.pkv_decode_line_wave_of.argtypes = [ctypes.c_int64, i32, ctypes.c_int64]
    L.pkv_decode_line_wave_of.restype = i32
    L.pkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.pkv_decode_workspace_bytes.restype = ctypes.c_size_t
    L.pkv_decode_workspace_bytes_split.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pkv_decode_workspace_bytes_split.restype = ctypes.c_size_t
    L.paged_decode_attention.argtypes = [vp, vp, vp, vp, i32p, i32p, i32, i32, i32, i32, i32, i32,
                                         i32, ctypes.c_float, i32, vp, ctypes.c_size_t, vp]
    L.paged_decode_attention.restype = i32
    L.paged_decode_attention_split.argtypes = [vp, vp, vp, vp, i32p, i32p, i32, i32, i32, i32,
                                               i32, i32, i32, ctypes.c_float, i32, i32, vp,
                                               ctypes.c_size_t, vp]
    L.paged_decode_attention_split.restype = i32
    L.paged_decode_attention_noalloc.argtypes = [vp, vp, vp, vp, i32p, i32p, i32, i32, i32, i32,
                                                 i32, i32, i32, ctypes.c_float, i32, vp]
    L.paged_decode_attention_noalloc.restype = i32
    L.paged_prefill_attention.argtypes = [vp, vp, i32p, vp, vp, i32p, i32p, i32, i32, i32, i32, i32,
                                          i32, i32, i32, ctypes.c_float, i32, vp]
    L.paged_prefill_attention.restype = i32
    L.kv_append_int8.argtypes = [vp, vp, i64p, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.kv_append_int8.restype = i32
    L.paged_decode_attention_int8.argtypes = [vp, vp, vp, vp, vp, vp, i32p, i32p, i32, i32, i32,
                                              i32, i32, i32, i32, ctypes.c_float, i32, vp,
                                              ctypes.c_size_t, vp]
    L.paged_decode_attention_int8.restype = i32
    L.paged_prefill_attention_int8.argtypes = [vp, vp, i32p, vp, vp, vp, vp, i32p, i32p, i32, i32,
                                               i32, i32, i32, i32, i32, i32, ctypes.c_float, vp]
    L.paged_prefill_attention_int8.restype = i32
    ptrs = ctypes.POINTER(ctypes.c_void_p)
    sizes = ctypes.POINTER(ctypes.c_int64)
    L.copy_blocks.argtypes = [ptrs, sizes, i32, i32, i32p, i32, vp]
    L.copy_blocks.restype = i32
    L.swap_blocks.argtypes = [ptrs, ptrs, sizes, i32, i32, i32, i32p, i32, vp]
    L.swap_blocks.restype = i32
    ip = ctypes.POINTER(ctypes.c_int)
    i64 = ctypes.c_int64
    L.pkv_bm_create.argtypes = [i32, i32, i32]
    L.pkv_bm_create.restype = vp
    L.pkv_bm_destroy.argtypes = [vp]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_add_sequence.argtypes = [vp, i64, vp, i32, vp, vp, ip, ip]
    L.pkv_bm_append.argtypes = [vp, i64, vp, i32, vp, vp, ip]
    L.pkv_bm_fork.argtypes = [vp, i64, i64]
    L.pkv_bm_free.argtypes = [vp, i64]
    L.pkv_bm_swap_out.argtypes = [vp, i64, vp, i32, ip]
    L.pkv_bm_swap_in.argtypes = [vp, i64, vp, i32, ip]
    L.pkv_bm_block_table.argtypes = [vp, i64, vp, i32, ip, ip]
    L.pkv_bm_get_stats.argtypes = [vp, ctypes.POINTER(BlockManagerStats)]
    L.pkv_bm_append_batch.argtypes = [vp, i32, vp, vp, vp, vp, ip]
    L.pkv_bm_block_tables.argtypes = [vp, i32, vp, vp, i32, vp]
    for f in ("pkv_bm_add_sequence", "pkv_bm_append", "pkv_bm_fork", "pkv_bm_free",
              "pkv_bm_swap_out", "pkv_bm_swap_in", "pkv_bm_block_table", "pkv_bm_get_stats",
              "pkv_bm_append_batch", "pkv_bm_block_tables"):
        getattr(L, f).restype = i32
    L.pkv_kv_cache_bytes.argtypes = [i32, i32, i32, i64, i64, i32, i32]
    L.pkv_kv_cache_bytes.restype = i64
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().pkv_status_string(int(status)).decode()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev(*ts: torch.Tensor):
    dev = ts[0].device
    for t in ts:
        _need(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
        _need(t.is_contiguous(), "all tensors must be contiguous")


def _pool_shape(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _need(k_cache.dim() == 4 and k_cache.shape[2] == 16, "pool must be [n_blocks, h_kv, 16, d_h]")
    _need(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "K/V pools differ")
    n_blocks, h_kv, _, d = k_cache.shape
    return int(n_blocks), int(h_kv), int(d)


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
              k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Write new K/V rows [T, h_kv, d_h] into pool slots (int64 [T]), in place."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _dev(k_new, v_new, slot_mapping, k_cache, v_cache)
    _need(k_new.dim() == 3 and k_new.shape[1:] == (h_kv, d) and v_new.shape == k_new.shape,
          "k_new/v_new must be [T, h_kv, d_h]")
    _need(k_new.dtype == k_cache.dtype == v_new.dtype, "dtype mismatch")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k_new.shape[0],),
          "slot_mapping must be int64 [T]")
    _need(k_cache.dtype in _DTYPE, f"unsupported dtype {k_cache.dtype}")
    rc = lib().kv_append(k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
                         k_cache.data_ptr(), v_cache.data_ptr(), int(k_new.shape[0]), h_kv, d,
                         n_blocks, _DTYPE[k_cache.dtype], _stream(k_cache))
    if rc != 0:
        raise PkvError("kv_append", rc)


def bind_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor):
    """kv_append with its arguments checked and marshalled once: returns a call
    that launches it (on the stream current now)."""
    kv_append(k_new[:0], v_new[:0], slot_mapping[:0], k_cache, v_cache)   # the checks
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(k_new.shape[0] == slot_mapping.shape[0] and v_new.shape == k_new.shape,
          "k_new/v_new/slot_mapping lengths differ")
    fn = lib().kv_append
    args = (k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), int(k_new.shape[0]), h_kv, d, n_blocks, _DTYPE[k_cache.dtype],
            _stream(k_cache))

    def call() -> None:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("kv_append", rc)
    return call


def decode_num_splits(B: int, h_q: int, h_kv: int, d_h: int, max_context_len: int,
                      dtype: torch.dtype = torch.bfloat16, num_splits: int = 0) -> int:
    """dtype: the pool's (torch.int8 for the INT8 cache)."""
    return int(lib().pkv_decode_num_splits(B, h_q, h_kv, d_h, max_context_len, _WS_DTYPE[dtype],
                                           num_splits))


def decode_line_start(total: int, splits: int, w: int) -> int:
    """First line position of decode wave w (pkv_decode_line_start); -1 if invalid."""
    return int(lib().pkv_decode_line_start(total, splits, w))


def decode_line_wave_of(total: int, splits: int, p: int) -> int:
    """The decode wave whose range holds line position p; -1 if invalid."""
    return int(lib().pkv_decode_line_wave_of(total, splits, p))


def decode_workspace_bytes(B: int, h_q: int, h_kv: int, d_h: int, max_context_len: int,
                           dtype: torch.dtype = torch.bfloat16, num_splits: int = 0) -> int:
    """Exact workspace of a decode call (pkv_decode_workspace_bytes_split).
    dtype: the pool's (torch.int8 for the INT8 cache)."""
    return int(lib().pkv_decode_workspace_bytes_split(B, h_q, h_kv, d_h, max_context_len,
                                                       _WS_DTYPE[dtype], num_splits))


def decode_workspace_bound(B: int, h_q: int, d_h: int, max_context_len: int) -> int:
    """Workspace that serves any automatic-split decode call of these sizes,
    whatever h_kv and dtype (pkv_decode_workspace_bytes)."""
    return int(lib().pkv_decode_workspace_bytes(B, h_q, d_h, max_context_len))


def _scale_pools(k_scale: torch.Tensor, v_scale: torch.Tensor, n_blocks: int, h_kv: int):
    _need(k_scale.dtype == torch.float32 and v_scale.dtype == torch.float32 and
          k_scale.shape == (n_blocks, h_kv, 16) and v_scale.shape == k_scale.shape and
          k_scale.is_contiguous() and v_scale.is_contiguous(),
          "k_scale/v_scale must be contiguous float32 [n_blocks, h_kv, 16]")


def kv_append_int8(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                   v_scale: torch.Tensor) -> None:
    """Quantise new K/V rows [T, h_kv, d_h] (bf16 or fp32) into the INT8 pools
    (int8 [n_blocks, h_kv, 16, d_h]) and their scales, in place."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(k_cache.dtype == torch.int8, "the INT8 pools must be int8")
    _scale_pools(k_scale, v_scale, n_blocks, h_kv)
    _dev(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)
    _need(k_new.dim() == 3 and k_new.shape[1:] == (h_kv, d) and v_new.shape == k_new.shape,
          "k_new/v_new must be [T, h_kv, d_h]")
    _need(k_new.dtype == v_new.dtype and k_new.dtype in _DTYPE, "k_new/v_new: bf16 or fp32")
    _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new/v_new must be contiguous")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k_new.shape[0],),
          "slot_mapping must be int64 [T]")
    rc = lib().kv_append_int8(k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
                              k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                              v_scale.data_ptr(), int(k_new.shape[0]), h_kv, d, n_blocks,
                              _DTYPE[k_new.dtype], _stream(k_cache))
    if rc != 0:
        raise PkvError("kv_append_int8", rc)


def bind_kv_append_int8(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                        v_scale: torch.Tensor):
    """kv_append_int8 with its arguments checked and marshalled once: returns a
    call that launches it (on the stream current now)."""
    kv_append_int8(k_new[:0], v_new[:0], slot_mapping[:0], k_cache, v_cache, k_scale,
                   v_scale)   # the checks
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(k_new.shape[0] == slot_mapping.shape[0] and v_new.shape == k_new.shape,
          "k_new/v_new/slot_mapping lengths differ")
    _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new/v_new must be contiguous")
    fn = lib().kv_append_int8
    args = (k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), int(k_new.shape[0]),
            h_kv, d, n_blocks, _DTYPE[k_new.dtype], _stream(k_cache))

    def call() -> None:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("kv_append_int8", rc)
    return call


def paged_decode_attention_int8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                k_scale: torch.Tensor, v_scale: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                max_context_len: int, scale: Optional[float] = None,
                                num_splits: int = 0, out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Single-token decode over the INT8 cache.  q, out: bf16 [B, h_q, d_h]."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(k_cache.dtype == torch.int8, "the INT8 pools must be int8")
    _scale_pools(k_scale, v_scale, n_blocks, h_kv)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == torch.bfloat16,
          "q must be bf16 [B, h_q, d_h]")
    B, h_q = int(q.shape[0]), int(q.shape[1])
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == B, "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,),
          "context_lens must be int32 [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _dev(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = decode_workspace_bytes(B, h_q, h_kv, d, int(max_context_len), torch.int8,
                                      num_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().paged_decode_attention_int8(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B, h_q, h_kv, d,
        n_blocks, int(block_tables.shape[1]), int(max_context_len), float(scale),
        int(num_splits), ws_ptr, ws_len, _stream(q))
    if rc != 0:
        raise PkvError("paged_decode_attention_int8", rc)
    return out


def bind_decode_int8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     k_scale: torch.Tensor, v_scale: torch.Tensor, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, max_context_len: int, out: torch.Tensor,
                     workspace: torch.Tensor, scale: Optional[float] = None,
                     num_splits: int = 0):
    """paged_decode_attention_int8 with its arguments checked and marshalled
    once (the first launch runs through the checked call): returns a call that
    launches it again on the same buffers (on the stream current now)."""
    paged_decode_attention_int8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                context_lens, max_context_len, scale=scale,
                                num_splits=num_splits, out=out, workspace=workspace)
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    B, h_q = int(q.shape[0]), int(q.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().paged_decode_attention_int8
    args = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            k_scale.data_ptr(), v_scale.data_ptr(), block_tables.data_ptr(),
            context_lens.data_ptr(), B, h_q, h_kv, d, n_blocks, int(block_tables.shape[1]),
            int(max_context_len), float(scale), int(num_splits), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(q))

    def call() -> torch.Tensor:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("paged_decode_attention_int8", rc)
        return out
    return call


def paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: Optional[float] = None,
                           num_splits: int = 0, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Single-token decode over paged K/V.  q, out: [B, h_q, d_h]."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == k_cache.dtype, "q must be [B, h_q, d_h]")
    B, h_q = int(q.shape[0]), int(q.shape[1])
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == B, "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,),
          "context_lens must be int32 [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _dev(q, k_cache, v_cache, block_tables, context_lens, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = decode_workspace_bytes(B, h_q, h_kv, d, int(max_context_len), q.dtype, num_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn, args = _decode_launch(out, q, k_cache, v_cache, block_tables, context_lens, B, h_q, h_kv,
                              d, n_blocks, max_context_len, scale, num_splits, ws_ptr, ws_len)
    rc = fn(*args)
    if rc != 0:
        raise PkvError("paged_decode_attention", rc)
    return out


def _decode_launch(out, q, k_cache, v_cache, block_tables, context_lens, B, h_q, h_kv, d,
                   n_blocks, max_context_len, scale, num_splits, ws_ptr, ws_len):
    """The C entry point and its arguments: paged_decode_attention for the
    automatic split, paged_decode_attention_split for an explicit count."""
    head = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), B, h_q, h_kv, d, n_blocks,
            int(block_tables.shape[1]), int(max_context_len), float(scale), _DTYPE[q.dtype])
    tail = (ws_ptr, ws_len, _stream(q))
    if int(num_splits) == 0:
        return lib().paged_decode_attention, head + tail
    return lib().paged_decode_attention_split, head + (int(num_splits),) + tail


def paged_decode_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, max_context_len: int,
                                   out: torch.Tensor, scale: Optional[float] = None) -> torch.Tensor:
    """paged_decode_attention through the entry point that allocates nothing
    (its workspace is the library's static device array).  out must be given:
    the binding allocates nothing either."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == k_cache.dtype, "q must be [B, h_q, d_h]")
    B, h_q = int(q.shape[0]), int(q.shape[1])
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == B, "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,),
          "context_lens must be int32 [B]")
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _dev(q, k_cache, v_cache, block_tables, context_lens, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = lib().paged_decode_attention_noalloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), B, h_q, h_kv, d, n_blocks,
        int(block_tables.shape[1]), int(max_context_len), float(scale), _DTYPE[q.dtype],
        _stream(q))
    if rc != 0:
        raise PkvError("paged_decode_attention_noalloc", rc)
    return out


def bind_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                out: torch.Tensor, workspace: torch.Tensor, scale: Optional[float] = None,
                num_splits: int = 0):
    """paged_decode_attention with its arguments checked and marshalled once
    (the first launch runs through the checked call): returns a call that
    launches it again on the same buffers (on the stream current now)."""
    paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                           scale=scale, num_splits=num_splits, out=out, workspace=workspace)
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    B, h_q = int(q.shape[0]), int(q.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn, args = _decode_launch(out, q, k_cache, v_cache, block_tables, context_lens, B, h_q, h_kv,
                              d, n_blocks, max_context_len, scale, num_splits,
                              workspace.data_ptr(), workspace.numel() * workspace.element_size())

    def call() -> torch.Tensor:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("paged_decode_attention", rc)
        return out
    return call


def paged_prefill_attention(q: torch.Tensor, cu_seqlens_q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, max_q_len: int,
                            scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal chunked prefill over paged K/V.  q, out: packed [T_q, h_q, d_h]."""
    return bind_prefill(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, max_q_len,
                        scale, out)()


def bind_prefill(q: torch.Tensor, cu_seqlens_q: torch.Tensor, k_cache: torch.Tensor,
                 v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                 max_q_len: int, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None):
    """Checks and marshals the arguments of paged_prefill_attention once and
    returns a call that launches it on them (on the stream current now), for
    loops that re-run one prefill on the same buffers.  The call returns out."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == k_cache.dtype,
          "q must be [T_q, h_q, d_h]")
    T_q, h_q = int(q.shape[0]), int(q.shape[1])
    S = int(context_lens.shape[0])
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.shape == (S + 1,),
          "cu_seqlens_q must be int32 [S + 1]")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == S, "block_tables must be int32 [S, max_blocks]")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32 [S]")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _dev(q, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().paged_prefill_attention
    args = (out.data_ptr(), q.data_ptr(), cu_seqlens_q.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), S, T_q,
            int(max_q_len), h_q, h_kv, d, n_blocks, int(block_tables.shape[1]), float(scale),
            _DTYPE[q.dtype], _stream(q))

    def call() -> torch.Tensor:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("paged_prefill_attention", rc)
        return out
    return call


def paged_prefill_attention_int8(q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                 k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 k_scale: torch.Tensor, v_scale: torch.Tensor,
                                 block_tables: torch.Tensor, context_lens: torch.Tensor,
                                 max_q_len: int, scale: Optional[float] = None,
                                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal chunked prefill over the INT8 cache.  q, out: bf16 packed [T_q, h_q, d_h]."""
    return bind_prefill_int8(q, cu_seqlens_q, k_cache, v_cache, k_scale, v_scale, block_tables,
                             context_lens, max_q_len, scale, out)()


def bind_prefill_int8(q: torch.Tensor, cu_seqlens_q: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, max_q_len: int,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None):
    """paged_prefill_attention_int8 with its arguments checked and marshalled
    once: returns a call that launches it (on the stream current now)."""
    n_blocks, h_kv, d = _pool_shape(k_cache, v_cache)
    _need(k_cache.dtype == torch.int8, "the INT8 pools must be int8")
    _scale_pools(k_scale, v_scale, n_blocks, h_kv)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == torch.bfloat16,
          "q must be bf16 [T_q, h_q, d_h]")
    T_q, h_q = int(q.shape[0]), int(q.shape[1])
    S = int(context_lens.shape[0])
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.shape == (S + 1,),
          "cu_seqlens_q must be int32 [S + 1]")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == S, "block_tables must be int32 [S, max_blocks]")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32 [S]")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _dev(q, cu_seqlens_q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    fn = lib().paged_prefill_attention_int8
    args = (out.data_ptr(), q.data_ptr(), cu_seqlens_q.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), block_tables.data_ptr(),
            context_lens.data_ptr(), S, T_q, int(max_q_len), h_q, h_kv, d, n_blocks,
            int(block_tables.shape[1]), float(scale), _stream(q))

    def call() -> torch.Tensor:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("paged_prefill_attention_int8", rc)
        return out
    return call


MAX_COPY_POOLS = 8


def _pool_set(pools, what: str):
    """(n_blocks, block bytes of each pool) of a pool set: tensors whose leading
    axis is the physical block."""
    _need(1 <= len(pools) <= MAX_COPY_POOLS, f"{what}: 1..{MAX_COPY_POOLS} pools")
    n_blocks = int(pools[0].shape[0])
    sizes = []
    for t in pools:
        _need(t.dim() >= 1 and int(t.shape[0]) == n_blocks,
              f"{what}: every pool needs the same number of blocks")
        _need(t.is_contiguous(), f"{what}: pools must be contiguous")
        _need(t.is_cuda or t.is_pinned(), f"{what}: pools must be on the GPU or in pinned memory")
        sizes.append(t.numel() * t.element_size() // n_blocks if n_blocks else 0)
    return n_blocks, sizes


def _pairs(pairs: torch.Tensor) -> int:
    _need(pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2 and
          pairs.is_contiguous(), "pairs must be contiguous int32 [n, 2] of (src, dst) blocks")
    _need(pairs.is_cuda or pairs.is_pinned(), "pairs must be on the GPU or in pinned memory")
    return int(pairs.shape[0])


def _copy_stream(tensors) -> int:
    for t in tensors:
        if t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def copy_blocks(pools, pairs: torch.Tensor) -> None:
    """Within one pool set (e.g. [k_cache, v_cache], plus the scale pools of an
    INT8 cache), block dst of every pool becomes a copy of block src, for every
    (src, dst) row of pairs (int32 [n, 2])."""
    bind_copy_blocks(pools, pairs)()


def bind_copy_blocks(pools, pairs: torch.Tensor):
    """copy_blocks with its arguments checked and marshalled once: returns a
    call that launches it (on the stream current now)."""
    n_blocks, sizes = _pool_set(pools, "pools")
    n = _pairs(pairs)
    ptr = (ctypes.c_void_p * len(pools))(*[t.data_ptr() for t in pools])
    bb = (ctypes.c_int64 * len(pools))(*sizes)
    fn = lib().copy_blocks
    args = (ptr, bb, len(pools), n_blocks, pairs.data_ptr(), n, _copy_stream([*pools, pairs]))

    def call() -> None:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("copy_blocks", rc)
    return call


def swap_blocks(src_pools, dst_pools, pairs: torch.Tensor) -> None:
    """Between two pool sets (GPU and pinned host, either way): block dst of
    dst_pools[i] becomes a copy of block src of src_pools[i]."""
    bind_swap_blocks(src_pools, dst_pools, pairs)()


def bind_swap_blocks(src_pools, dst_pools, pairs: torch.Tensor):
    """swap_blocks with its arguments checked and marshalled once."""
    _need(len(src_pools) == len(dst_pools), "pool sets differ in length")
    n_src, s_sizes = _pool_set(src_pools, "src_pools")
    n_dst, d_sizes = _pool_set(dst_pools, "dst_pools")
    for s, d in zip(src_pools, dst_pools):
        _need(s.shape[1:] == d.shape[1:] and s.dtype == d.dtype,
              "a source and a destination pool differ in block shape or dtype")
    n = _pairs(pairs)
    sp = (ctypes.c_void_p * len(src_pools))(*[t.data_ptr() for t in src_pools])
    dp = (ctypes.c_void_p * len(dst_pools))(*[t.data_ptr() for t in dst_pools])
    bb = (ctypes.c_int64 * len(src_pools))(*s_sizes)
    fn = lib().swap_blocks
    args = (sp, dp, bb, len(src_pools), n_src, n_dst, pairs.data_ptr(), n,
            _copy_stream([*src_pools, *dst_pools, pairs]))

    def call() -> None:
        rc = fn(*args)
        if rc != 0:
            raise PkvError("swap_blocks", rc)
    return call


def kv_cache_bytes(n_layers: int, h_kv: int, d_h: int, batch: int, seq_len: int,
                   dtype: torch.dtype = torch.bfloat16, paged: bool = False) -> int:
    """KV-cache footprint in bytes (torch.int8: the INT8 cache with its scales)."""
    r = lib().pkv_kv_cache_bytes(n_layers, h_kv, d_h, batch, seq_len, _WS_DTYPE[dtype],
                                 int(paged))
    if r < 0:
        raise ValueError("invalid kv_cache_bytes arguments")
    return int(r)


class BlockManager:
    """The library's block manager (host-only C++): block tables, slots, prefix
    cache, copy on write and swap plans.  Token ids are int32; slots come back
    as int64 arrays ready for kv_append (-1 = already cached), copy pairs as
    int32 [n, 2] arrays ready for copy_blocks / swap_blocks."""

    def __init__(self, n_blocks: int, n_host_blocks: int = 0, prefix_cache: bool = True):
        self._L = lib()
        self._h = self._L.pkv_bm_create(int(n_blocks), int(n_host_blocks), int(prefix_cache))
        if not self._h:
            raise ValueError("pkv_bm_create: invalid sizes or out of memory")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._L.pkv_bm_destroy(h)

    def _check(self, what: str, rc: int):
        if rc == PKV_ERR_NO_BLOCKS:
            raise NoBlocksError(what, rc)
        if rc != 0:
            raise PkvError(what, rc)

    @staticmethod
    def _tokens(tokens) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))

    def add_sequence(self, seq_id: int, tokens):
        """-> (n_cached, slots int64 [n], cow_pairs int32 [0 or 1, 2])"""
        t = self._tokens(tokens)
        slots = np.empty(len(t), np.int64)
        cow = np.empty((1, 2), np.int32)
        n_cow, n_cached = ctypes.c_int(0), ctypes.c_int(0)
        self._check("pkv_bm_add_sequence", self._L.pkv_bm_add_sequence(
            self._h, int(seq_id), t.ctypes.data, len(t), slots.ctypes.data, cow.ctypes.data,
            ctypes.byref(n_cow), ctypes.byref(n_cached)))
        return n_cached.value, slots, cow[:n_cow.value].copy()

    def append(self, seq_id: int, tokens):
        """-> (slots int64 [n], cow_pairs int32 [0 or 1, 2])"""
        t = self._tokens(tokens)
        slots = np.empty(len(t), np.int64)
        cow = np.empty((1, 2), np.int32)
        n_cow = ctypes.c_int(0)
        self._check("pkv_bm_append", self._L.pkv_bm_append(
            self._h, int(seq_id), t.ctypes.data, len(t), slots.ctypes.data, cow.ctypes.data,
            ctypes.byref(n_cow)))
        return slots, cow[:n_cow.value].copy()

    def append_batch(self, seq_ids, tokens):
        """One token per sequence (a decode step) -> (slots int64 [n],
        cow_pairs int32 [k, 2])"""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        t = self._tokens(tokens)
        _need(len(ids) == len(t), "one token per sequence")
        slots = np.empty(len(t), np.int64)
        cow = np.empty((max(len(t), 1), 2), np.int32)
        n_cow = ctypes.c_int(0)
        self._check("pkv_bm_append_batch", self._L.pkv_bm_append_batch(
            self._h, len(t), ids.ctypes.data, t.ctypes.data, slots.ctypes.data, cow.ctypes.data,
            ctypes.byref(n_cow)))
        return slots, cow[:n_cow.value].copy()

    def block_tables(self, seq_ids, max_blocks: Optional[int] = None):
        """-> (tables int32 [n, max_blocks], context_lens int32 [n]) for the
        attention calls; max_blocks defaults to the longest table."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))
        if max_blocks is None:
            max_blocks = max([len(self.block_table(int(i))[0]) for i in ids] + [1])
        tables = np.empty((len(ids), max_blocks), np.int32)
        lens = np.empty(len(ids), np.int32)
        self._check("pkv_bm_block_tables", self._L.pkv_bm_block_tables(
            self._h, len(ids), ids.ctypes.data, tables.ctypes.data, max_blocks,
            lens.ctypes.data))
        return tables, lens

    def fork(self, parent: int, child: int) -> None:
        self._check("pkv_bm_fork", self._L.pkv_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq_id: int) -> None:
        self._check("pkv_bm_free", self._L.pkv_bm_free(self._h, int(seq_id)))

    def _swap(self, fn, what, seq_id):
        n_blocks, length = ctypes.c_int(0), ctypes.c_int(0)
        self._L.pkv_bm_block_table(self._h, int(seq_id), None, 0, ctypes.byref(n_blocks),
                                   ctypes.byref(length))
        cap = max(n_blocks.value, 1)
        pairs = np.empty((cap, 2), np.int32)
        n = ctypes.c_int(0)
        self._check(what, fn(self._h, int(seq_id), pairs.ctypes.data, cap, ctypes.byref(n)))
        return pairs[:n.value].copy()

    def swap_out(self, seq_id: int) -> np.ndarray:
        """-> (device block, host block) pairs int32 [n, 2]"""
        return self._swap(self._L.pkv_bm_swap_out, "pkv_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int) -> np.ndarray:
        """-> (host block, device block) pairs int32 [n, 2]"""
        return self._swap(self._L.pkv_bm_swap_in, "pkv_bm_swap_in", seq_id)

    def block_table(self, seq_id: int):
        """-> (block ids int32 [n_blocks], sequence length)"""
        n_blocks, length = ctypes.c_int(0), ctypes.c_int(0)
        rc = self._L.pkv_bm_block_table(self._h, int(seq_id), None, 0, ctypes.byref(n_blocks),
                                        ctypes.byref(length))
        if rc != 0 and n_blocks.value == 0:
            self._check("pkv_bm_block_table", rc)
        table = np.empty(max(n_blocks.value, 1), np.int32)
        self._check("pkv_bm_block_table", self._L.pkv_bm_block_table(
            self._h, int(seq_id), table.ctypes.data, len(table), ctypes.byref(n_blocks),
            ctypes.byref(length)))
        return table[:n_blocks.value].copy(), length.value

    def stats(self) -> dict:
        st = BlockManagerStats()
        self._check("pkv_bm_get_stats", self._L.pkv_bm_get_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in BlockManagerStats._fields_}
