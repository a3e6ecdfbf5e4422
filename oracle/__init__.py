"""CPU oracle for paged MLA decode with split-KV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it, and it never loads the product path.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp64, OpenMP over query
rows); this module only compiles it with gcc and marshals numpy arrays.

Functions and the passages they follow (pages on FlashMLA):

* :func:`decode` -- the definition of the decode: per query row, scores over
  the row's visible keys of the paged cache, softmax, weighted sum of the
  first 512 dims of the same cached rows, plus the log-sum-exp.  Head dim 576,
  value dim 512 and Shared-KV come from "DeepSeek 开源记-第1天-FlashMLA",
  section 2; paging with block size 64 and BF16 from the ygpos news page; the
  call shape from section 6 of the cnblogs page.
* :func:`decode_split` -- the same attention evaluated piecewise on cut key
  ranges and merged by log-sum-exp (the "output merge" step, section 4 of the
  cnblogs page).
* :func:`schedule` -- the split-KV partition rule of the metadata call (block
  scheduling, section 3.1 of the jsxs2 explainer); the rule itself is a
  reading documented in the C file.

Pins: every function is checked against something other than itself in
``tests/test_oracle_pins.py`` (dense float64 brute force, closed forms,
invariants, a library routine on special cases, brute-force enumeration).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")
_lib = None

D = 576
DV = 512
PAGE = 64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.mla_oracle_decode.argtypes = [p, p, p, p, i, i, i, i, i, i, i, i, i, i,
                                          ctypes.c_double, i, p, p]
        lib.mla_oracle_decode.restype = i
        lib.mla_oracle_decode_split.argtypes = [p, p, p, p, i, i, i, i, i, i, i, i, i, i,
                                                ctypes.c_double, i, p, p, p, p]
        lib.mla_oracle_widen.argtypes = [p, ctypes.c_long, i, p]
        lib.mla_oracle_widen.restype = i
        lib.mla_oracle_decode_split.restype = i
        lib.mla_oracle_schedule.argtypes = [p, i, i, i, i, p, p]
        lib.mla_oracle_schedule.restype = i
        lib.mla_oracle_num_threads.argtypes = []
        lib.mla_oracle_num_threads.restype = i
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().mla_oracle_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _prep(q, kcache, block_table, seqlens):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kcache = np.ascontiguousarray(kcache, dtype=np.uint16)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    if q.ndim != 4 or kcache.ndim != 4 or block_table.ndim != 2 or seqlens.ndim != 1:
        raise ValueError("q [B,s_q,h_q,d], kcache [P,page,h_kv,d], block_table [B,max_blocks], "
                         "seqlens [B] expected")
    B, s_q, h_q, d = q.shape
    num_pages, page, h_kv, d2 = kcache.shape
    if d2 != d or block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("shape mismatch between q, kcache, block_table and seqlens")
    return q, kcache, block_table, seqlens, (B, s_q, h_q, d, num_pages, page, h_kv)


_DTYPES = {"bf16": 0, "fp16": 1}


def widen(bits, dtype: str = "bf16"):
    """The float64 values of 16-bit bit patterns (uint16) of type ``dtype``."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.zeros(bits.shape, dtype=np.float64)
    rc = _load().mla_oracle_widen(_ptr(bits), int(bits.size), _DTYPES[dtype], _ptr(out))
    if rc != 0:
        raise ValueError(f"mla_oracle_widen failed with code {rc}")
    return out


def decode(q, kcache, block_table, seqlens, *, causal: bool, scale: float, dv: int = DV,
           dtype: str = "bf16"):
    """Reference decode in float64.

    ``q``: 16-bit bits uint16 [B, s_q, h_q, d] of type ``dtype`` ("bf16" or
    "fp16"); ``kcache``: same type, uint16 [num_pages, page, h_kv, d]; ``block_table``: int32 [B, max_blocks];
    ``seqlens``: int32 [B].  Returns ``(out [B, s_q, h_q, dv] float64,
    lse [B, s_q, h_q] float64)``; empty rows give out 0 and lse -inf.
    """
    q, kcache, block_table, seqlens, (B, s_q, h_q, d, P, page, h_kv) = _prep(
        q, kcache, block_table, seqlens)
    out = np.zeros((B, s_q, h_q, dv), dtype=np.float64)
    lse = np.zeros((B, s_q, h_q), dtype=np.float64)
    rc = _load().mla_oracle_decode(_ptr(q), _ptr(kcache), _ptr(block_table), _ptr(seqlens), B, s_q,
                                   h_q, h_kv, d, dv, page, P, block_table.shape[1], int(causal),
                                   float(scale), _DTYPES[dtype], _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"mla_oracle_decode failed with code {rc}")
    return out, lse


def decode_split(q, kcache, block_table, seqlens, cuts, *, causal: bool, scale: float,
                 dv: int = DV, dtype: str = "bf16"):
    """Piecewise decode merged by log-sum-exp.

    ``cuts``: list (length B) of ascending interior cut positions (token
    indices strictly between 0 and N_b) for each sequence.
    """
    q, kcache, block_table, seqlens, (B, s_q, h_q, d, P, page, h_kv) = _prep(
        q, kcache, block_table, seqlens)
    if len(cuts) != B:
        raise ValueError("one cut list per sequence expected")
    cut_ptr = np.zeros(B + 1, dtype=np.int32)
    for b, c in enumerate(cuts):
        cut_ptr[b + 1] = cut_ptr[b] + len(c)
    flat = np.ascontiguousarray(
        np.concatenate([np.asarray(c, dtype=np.int32) for c in cuts]) if cut_ptr[-1] > 0
        else np.zeros(1, dtype=np.int32), dtype=np.int32)
    out = np.zeros((B, s_q, h_q, dv), dtype=np.float64)
    lse = np.zeros((B, s_q, h_q), dtype=np.float64)
    rc = _load().mla_oracle_decode_split(_ptr(q), _ptr(kcache), _ptr(block_table), _ptr(seqlens),
                                         B, s_q, h_q, h_kv, d, dv, page, P, block_table.shape[1],
                                         int(causal), float(scale), _DTYPES[dtype], _ptr(cut_ptr),
                                         _ptr(flat),
                                         _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"mla_oracle_decode_split failed with code {rc}")
    return out, lse


def schedule(seqlens, *, num_parts: int, fixed_cost: int, unit_tokens: int = 32):
    """Split-KV partition: returns ``(tile_meta int32 [num_parts, 8],
    num_splits int32 [B+1])`` following the rule written out in the C file.
    Sequences are cut only at multiples of ``unit_tokens`` keys."""
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    B = seqlens.shape[0]
    meta = np.zeros((num_parts, 8), dtype=np.int32)
    splits = np.zeros(B + 1, dtype=np.int32)
    rc = _load().mla_oracle_schedule(_ptr(seqlens), B, unit_tokens, num_parts, fixed_cost,
                                     _ptr(meta), _ptr(splits))
    if rc != 0:
        raise ValueError(f"mla_oracle_schedule failed with code {rc}")
    return meta, splits
