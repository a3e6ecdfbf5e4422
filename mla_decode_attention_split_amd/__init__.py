"""Paged MLA decode with split-KV on MI355X (gfx950).

Thin binding over ``libmla_decode.so`` (C ABI in ``include/mla_decode.h``):
argument marshalling only -- every step of the decode runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.

Entry points with the C names: :func:`mla_metadata_shape`,
:func:`mla_tile_shape`, :func:`mla_get_metadata` (the C calls
``mla_get_metadata`` / ``mla_get_metadata_ex``), :func:`mla_workspace_bytes`,
:func:`mla_decode`, :func:`mla_decode_splitkv`, :func:`mla_decode_combine`.  The two calls the pages show ("DeepSeek 开源记-第1天-
FlashMLA", section 6) are :func:`get_mla_metadata` and
:func:`flash_mla_with_kvcache`, with the same argument order.

If the library is missing or cannot be loaded, every call raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import sys

__all__ = [
    "MlaError", "library_path", "mla_metadata_shape", "mla_tile_shape", "mla_get_metadata",
    "mla_workspace_bytes", "mla_decode", "mla_decode_splitkv", "mla_decode_combine",
    "mla_decode_noalloc",
    "get_mla_metadata", "flash_mla_with_kvcache",
    "HEAD_DIM", "VALUE_DIM", "PAGE_SIZE",
]

HEAD_DIM = 576
VALUE_DIM = 512
DTYPE_BF16, DTYPE_FP16 = 0, 1  # element types of q, the cache and out (mla_decode.h)
PAGE_SIZE = 64
METADATA_WORDS = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmla_decode.so")
_lib = None


class MlaError(RuntimeError):
    """A nonzero status from the C library (message from mla_last_error)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MlaError(-4, f"{_LIB_PATH} is missing: build it with "
                           "`python -m mla_decode_attention_split_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i, p, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.mla_status_string.argtypes = [i]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    pi = ctypes.POINTER(i)
    lib.mla_metadata_shape.argtypes = [i, i, i, pi, pi]
    lib.mla_metadata_shape.restype = i
    lib.mla_tile_shape.argtypes = [i, i, pi, pi, pi]
    lib.mla_tile_shape.restype = i
    lib.mla_get_metadata.argtypes = [p, i, i, i, p, p, p]
    lib.mla_get_metadata.restype = i
    lib.mla_get_metadata_ex.argtypes = [p, i, i, i, p, p, p, i, i]
    lib.mla_get_metadata_ex.restype = i
    lib.mla_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.mla_workspace_bytes.restype = sz
    decode_args = [p, p, p, p, i, i, i, i, i, i, i, i, i, i, p, i, p, i, ctypes.c_float, p, p, p,
                   sz, p]
    lib.mla_decode.argtypes = decode_args
    lib.mla_decode.restype = i
    lib.mla_decode_splitkv.argtypes = decode_args
    lib.mla_decode_splitkv.restype = i
    lib.mla_decode_combine.argtypes = [p, i, i, i, i, i, i, p, p, p, sz, p]
    lib.mla_decode_combine.restype = i
    lib.mla_decode_noalloc.argtypes = decode_args[:-3] + [p]
    lib.mla_decode_noalloc.restype = i
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = _load()
        raise MlaError(status, (lib.mla_last_error() or lib.mla_status_string(status)).decode())


def _stream_of(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mla_metadata_shape(batch: int, q_rows_per_kv_head: int, h_kv: int):
    """Returns ``(num_parts, words_per_part)`` of the default partition on the
    current device: ``tile_metadata`` is int32 ``[num_parts, words_per_part]``."""
    lib = _load()
    n, wpp = ctypes.c_int(), ctypes.c_int()
    _check(lib.mla_metadata_shape(int(batch), int(q_rows_per_kv_head), int(h_kv), ctypes.byref(n),
                                  ctypes.byref(wpp)))
    return n.value, wpp.value


def mla_tile_shape(q_rows_per_kv_head: int, h_kv: int):
    """Returns ``(tile_rows, m_tiles, fixed_cost)``: the decode kernel's row tile
    for this many rows per KV head and the partition's default per-sequence
    cost (32-key units)."""
    lib = _load()
    t, m, f = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib.mla_tile_shape(int(q_rows_per_kv_head), int(h_kv), ctypes.byref(t), ctypes.byref(m),
                              ctypes.byref(f)))
    return t.value, m.value, f.value


def mla_get_metadata(cache_seqlens, q_rows_per_kv_head: int, h_kv: int, *,
                     num_parts: int | None = None, fixed_cost: int | None = None,
                     tile_metadata=None, num_splits=None):
    """Split-KV scheduling metadata on the device of ``cache_seqlens``.

    Returns ``(tile_metadata int32 [num_parts, 8], num_splits int32 [B+1])``.
    ``num_parts`` / ``fixed_cost`` override the library's defaults (the C call
    ``mla_get_metadata_ex``); without them this is ``mla_get_metadata``.
    Preallocated output tensors may be passed in.
    """
    import torch
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda or cache_seqlens.dim() != 1:
        raise ValueError("cache_seqlens must be a 1-D int32 CUDA tensor")
    seqlens = cache_seqlens.contiguous()
    batch = seqlens.shape[0]
    with torch.cuda.device(seqlens.device):
        parts = int(num_parts) if num_parts is not None else \
            mla_metadata_shape(batch, q_rows_per_kv_head, h_kv)[0]
        meta = tile_metadata
        if meta is None:
            meta = torch.empty((parts, METADATA_WORDS), dtype=torch.int32, device=seqlens.device)
        elif (meta.dtype != torch.int32 or tuple(meta.shape) != (parts, METADATA_WORDS)
              or not meta.is_contiguous()):
            raise ValueError("tile_metadata must be contiguous int32 [num_parts, 8]")
        splits = num_splits
        if splits is None:
            splits = torch.empty((batch + 1,), dtype=torch.int32, device=seqlens.device)
        elif splits.dtype != torch.int32 or tuple(splits.shape) != (batch + 1,):
            raise ValueError("num_splits must be int32 [B+1]")
        lib = _load()
        stream = _stream_of(seqlens.device)
        if num_parts is None and fixed_cost is None:
            _check(lib.mla_get_metadata(seqlens.data_ptr(), batch, int(q_rows_per_kv_head),
                                        int(h_kv), meta.data_ptr(), splits.data_ptr(), stream))
        else:
            _check(lib.mla_get_metadata_ex(seqlens.data_ptr(), batch, int(q_rows_per_kv_head),
                                           int(h_kv), meta.data_ptr(), splits.data_ptr(), stream,
                                           parts if num_parts is not None else 0,
                                           int(fixed_cost) if fixed_cost is not None else 0))
        if os.environ.get("MLA_DECODE_LOG", "0") not in ("", "0"):
            # debugging aid only: this reads num_splits back (a device sync)
            pieces = (splits[1:] - splits[:-1]).cpu()
            print(f"[mla] split stats: {int(pieces.sum())} pieces over {batch} sequences, "
                  f"max {int(pieces.max())}, split sequences {int((pieces > 1).sum())}",
                  file=sys.stderr, flush=True)
    return meta, splits


def mla_workspace_bytes(batch: int, q_rows_per_kv_head: int, h_kv: int, num_parts: int,
                        dv: int = VALUE_DIM) -> int:
    return int(_load().mla_workspace_bytes(int(batch), int(q_rows_per_kv_head), int(h_kv),
                                           int(num_parts), int(dv)))


def _decode_call(fn_name, q, blocked_k, block_table, cache_seqlens, tile_metadata, num_splits,
                 causal, softmax_scale, out, lse, workspace):
    import torch
    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}
    if q.dtype not in dtypes or blocked_k.dtype != q.dtype:
        raise ValueError("q and blocked_k must both be bfloat16 or both float16")
    dtype = dtypes[q.dtype]
    if block_table.dtype != torch.int32 or cache_seqlens.dtype != torch.int32:
        raise ValueError("block_table and cache_seqlens must be int32")
    if tile_metadata.dtype != torch.int32 or num_splits.dtype != torch.int32:
        raise ValueError("tile_metadata and num_splits must be int32")
    for name, t in (("q", q), ("blocked_k", blocked_k), ("block_table", block_table),
                    ("cache_seqlens", cache_seqlens), ("tile_metadata", tile_metadata),
                    ("num_splits", num_splits)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if q.dim() != 4 or blocked_k.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q [B,s_q,h_q,d], blocked_k [P,page,h_kv,d], block_table [B,n] expected")
    B, s_q, h_q, d = q.shape
    num_pages, page, h_kv, d2 = blocked_k.shape
    if d2 != d:
        raise ValueError("q and blocked_k disagree on the head dim")
    if block_table.shape[0] != B or cache_seqlens.shape != (B,):
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if tile_metadata.dim() != 2 or tile_metadata.shape[1] != METADATA_WORDS:
        raise ValueError("tile_metadata must be [num_parts, 8]")
    if num_splits.shape != (B + 1,):
        raise ValueError("num_splits must be [B+1]")
    num_parts = tile_metadata.shape[0]
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    dev = q.device
    M = s_q * h_q // max(h_kv, 1)
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, s_q, h_q, VALUE_DIM), dtype=q.dtype, device=dev)
        elif out.dtype != q.dtype:
            raise ValueError("out must have q's dtype")
        if lse is None:
            lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
        need = mla_workspace_bytes(B, M, h_kv, num_parts) if h_q % max(h_kv, 1) == 0 else 0
        if workspace is None:
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        fn = getattr(_load(), fn_name)
        _check(fn(q.data_ptr(), blocked_k.data_ptr(), block_table.data_ptr(),
                  cache_seqlens.data_ptr(), B, s_q, h_q, h_kv, d, VALUE_DIM, dtype, num_pages, page,
                  block_table.shape[1], tile_metadata.data_ptr(), num_parts, num_splits.data_ptr(),
                  int(bool(causal)), scale, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                  workspace.numel() * workspace.element_size(), _stream_of(dev)))
    return out, lse, workspace


def mla_decode(q, blocked_k, block_table, cache_seqlens, tile_metadata, num_splits, *,
               causal: bool = False, softmax_scale: float | None = None, out=None, lse=None,
               workspace=None):
    """Paged MLA decode.  ``q`` bf16 [B, s_q, h_q, 576]; ``blocked_k`` bf16
    [num_pages, 64, h_kv, 576]; ``block_table`` int32 [B, max_blocks];
    ``cache_seqlens`` int32 [B].  Returns ``(out bf16 [B, s_q, h_q, 512],
    lse fp32 [B, s_q, h_q])``."""
    out, lse, _ = _decode_call("mla_decode", q, blocked_k, block_table, cache_seqlens,
                               tile_metadata, num_splits, causal, softmax_scale, out, lse,
                               workspace)
    return out, lse


def mla_decode_noalloc(q, blocked_k, block_table, cache_seqlens, tile_metadata, num_splits, *,
                       causal: bool = False, softmax_scale: float | None = None, out=None, lse=None):
    """:func:`mla_decode` without a workspace: the split partials go to the
    library's own device scratch (C call ``mla_decode_noalloc``), for callers
    that cannot allocate device memory.  Pass ``out`` and ``lse`` to keep the
    call free of allocations here too."""
    import torch
    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}
    if q.dtype not in dtypes or blocked_k.dtype != q.dtype:
        raise ValueError("q and blocked_k must both be bfloat16 or both float16")
    for name, t in (("q", q), ("blocked_k", blocked_k), ("block_table", block_table),
                    ("cache_seqlens", cache_seqlens), ("tile_metadata", tile_metadata),
                    ("num_splits", num_splits)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if q.dim() != 4 or blocked_k.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q [B,s_q,h_q,d], blocked_k [P,page,h_kv,d], block_table [B,n] expected")
    B, s_q, h_q, d = q.shape
    num_pages, page, h_kv, _ = blocked_k.shape
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    dev = q.device
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, s_q, h_q, VALUE_DIM), dtype=q.dtype, device=dev)
        elif out.dtype != q.dtype:
            raise ValueError("out must have q's dtype")
        if lse is None:
            lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
        _check(_load().mla_decode_noalloc(
            q.data_ptr(), blocked_k.data_ptr(), block_table.data_ptr(), cache_seqlens.data_ptr(), B,
            s_q, h_q, h_kv, d, VALUE_DIM, dtypes[q.dtype], num_pages, page, block_table.shape[1],
            tile_metadata.data_ptr(), tile_metadata.shape[0], num_splits.data_ptr(),
            int(bool(causal)), scale, out.data_ptr(), lse.data_ptr(), _stream_of(dev)))
    return out, lse


def mla_decode_splitkv(q, blocked_k, block_table, cache_seqlens, tile_metadata, num_splits, *,
                       causal: bool = False, softmax_scale: float | None = None, out=None,
                       lse=None, workspace=None):
    """Main kernel only; returns ``(out, lse, workspace)`` -- pass the same
    ``out``, ``lse`` and ``workspace`` to :func:`mla_decode_combine`."""
    return _decode_call("mla_decode_splitkv", q, blocked_k, block_table, cache_seqlens,
                        tile_metadata, num_splits, causal, softmax_scale, out, lse, workspace)


def mla_decode_combine(num_splits, out, lse, workspace, *, num_parts: int, h_kv: int = 1):
    """Merge the split partials left by :func:`mla_decode_splitkv`."""
    import torch
    B, s_q, h_q, _ = out.shape
    dtype = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}[out.dtype]
    with _torch_device(out.device):
        _check(_load().mla_decode_combine(
            num_splits.data_ptr(), B, s_q, h_q, int(h_kv), int(num_parts), dtype, out.data_ptr(),
            lse.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_of(out.device)))
    return out, lse


def _torch_device(dev):
    import torch
    return torch.cuda.device(dev)


def get_mla_metadata(cache_seqlens, num_heads_per_head_k: int, num_heads_k: int):
    """The pages' metadata call (cnblogs page, section 6): the cache lengths,
    the query rows per KV head and the KV head count in; the scheduling
    metadata and the per-sequence split counts out."""
    return mla_get_metadata(cache_seqlens, num_heads_per_head_k, num_heads_k)


def flash_mla_with_kvcache(q, k_cache, block_table, cache_seqlens, head_dim_v: int,
                           tile_scheduler_metadata, num_splits, softmax_scale=None,
                           causal: bool = False):
    """The pages' decode call; returns ``(output, lse)``."""
    if head_dim_v != VALUE_DIM:
        raise MlaError(-2, f"value dim {head_dim_v} (only {VALUE_DIM})")
    return mla_decode(q, k_cache, block_table, cache_seqlens, tile_scheduler_metadata, num_splits,
                      causal=causal, softmax_scale=softmax_scale)
