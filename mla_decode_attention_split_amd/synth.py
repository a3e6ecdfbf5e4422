"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic.  Both the HIP path and the CPU oracle consume what
it produces (bf16 or fp16 values are carried as their uint16 bit patterns).

Shapes follow the pages' call (q, blocked_k, block_table, cache_seqlens) and
their fixed sizes: row width 576 = 512 latent + 64 rope, page of 64 tokens,
bf16 storage.  The named workloads are:

* ``tiny``     B=2, s_q=1, h_q=16, N=[64, 200]; block_table [2, 4] is a random
               permutation of the 8 physical pages of the pool.
* ``membound`` B=32, s_q=1, h_q=16, every N=4096, pool of 2048 pages.
* ``mtp``      B=64, s_q=2 causal, h_q=128, N ~ Uniform{1024..8192}.
* ``large``    B=128, s_q=1, h_q=128, every N=4096, pool of 8192 pages.
* ``ragged``   B=16, s_q=1, h_q=64, N = clip(rint(lognormal(ln 2048, 1)),
               1, 32768) with N[0] = N[8] = 32768.

* ``hkv2``     B=32, s_q=1, h_q=32, h_kv=2, every N=4096.

Values: q and every cache page (used or not) are N(0, 1) drawn in float32
and rounded to bf16 (or, with ``dtype="fp16"``, to fp16), round to nearest
even.  block_table is a seeded
permutation of the pool laid out row-major over the pages each sequence
needs; unused table entries point at ``pad_page``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 576
DV = 512
PAGE = 64
BF16_NAN = np.uint16(0x7FC0)
F16_NAN = np.uint16(0x7E00)

WORKLOADS = ("tiny", "membound", "mtp", "large", "ragged", "hkv2")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _normal_16bit(rng: np.random.Generator, shape, chunk: int = 1 << 24,
                 dtype: str = "bf16") -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = bf16_bits(x) if dtype == "bf16" else x.astype(np.float16).view(np.uint16)
    return out.reshape(shape)


@dataclass
class Workload:
    name: str
    q: np.ndarray            # uint16 [B, s_q, h_q, D]
    kcache: np.ndarray       # uint16 [num_pages, PAGE, h_kv, D]
    block_table: np.ndarray  # int32  [B, max_blocks]
    seqlens: np.ndarray      # int32  [B]
    s_q: int
    h_q: int
    h_kv: int
    causal: bool
    scale: float
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"      # element type of q and kcache: "bf16" or "fp16"

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    @property
    def rows_per_kv_head(self) -> int:
        return self.s_q * self.h_q // self.h_kv


def make_workload(seqlens, *, s_q: int = 1, h_q: int = 16, h_kv: int = 1, causal: bool = False,
                  seed: int = 0, extra_pages: int = 0, table_width: int | None = None,
                  pad: str = "valid", poison_tail: bool = False, name: str = "custom",
                  scale: float | None = None, dtype: str = "bf16") -> Workload:
    """Paged workload for the given sequence lengths.

    ``pad``: what unused block_table entries hold -- ``"valid"`` (page 0 of
    the pool, a legal index), ``"poison"`` (an extra NaN-filled page appended
    to the pool) or ``"minus1"`` (-1; oracle-only inputs).
    ``poison_tail``: fill cache rows past N in each sequence's last page, and
    every page no sequence uses, with NaN.
    """
    rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    B = seqlens.shape[0]
    pages_needed = (seqlens.astype(np.int64) + PAGE - 1) // PAGE
    used = int(pages_needed.sum())
    pool = used + extra_pages
    width = int(max(1, pages_needed.max() if B else 1)) if table_width is None else table_width
    if width < (pages_needed.max() if B else 0):
        raise ValueError("table_width smaller than the pages a sequence needs")
    perm = rng.permutation(pool).astype(np.int32)
    if dtype not in ("bf16", "fp16"):
        raise ValueError("dtype must be bf16 or fp16")
    nan = BF16_NAN if dtype == "bf16" else F16_NAN
    q = _normal_16bit(rng, (B, s_q, h_q, D), dtype=dtype)
    kcache = _normal_16bit(rng, (pool + (1 if pad == "poison" else 0), PAGE, h_kv, D), dtype=dtype)
    pad_val = {"valid": 0, "poison": pool, "minus1": -1}[pad]
    table = np.full((B, width), pad_val, dtype=np.int32)
    off = 0
    for b in range(B):
        r = int(pages_needed[b])
        table[b, :r] = perm[off:off + r]
        off += r
    if pad == "poison":
        kcache[pool] = nan
    if poison_tail:
        for b in range(B):
            n = int(seqlens[b])
            if n % PAGE:
                kcache[table[b, n // PAGE], n % PAGE:] = nan
        for p in perm[used:]:
            kcache[p] = nan
    return Workload(name=name, q=q, kcache=kcache, block_table=table, seqlens=seqlens, s_q=s_q,
                    h_q=h_q, h_kv=h_kv, causal=causal,
                    scale=float(D ** -0.5) if scale is None else float(scale),
                    meta={"seed": seed, "pool_pages": pool}, dtype=dtype)


def named_workload(name: str, seed: int | None = None, dtype: str = "bf16") -> Workload:
    """One of the named workloads (seed defaults to its index); ``dtype``
    "fp16" draws the same shapes in fp16 (tiny is bf16 only)."""
    idx = WORKLOADS.index(name)
    seed = idx if seed is None else seed
    kw = {"dtype": dtype}
    if name == "tiny":
        if dtype != "bf16":
            raise ValueError("the tiny workload is bf16 only")
        rng = np.random.default_rng(seed)
        perm = rng.permutation(8).astype(np.int32)
        q = _normal_16bit(rng, (2, 1, 16, D))
        kcache = _normal_16bit(rng, (8, PAGE, 1, D))
        return Workload(name=name, q=q, kcache=kcache, block_table=perm.reshape(2, 4).copy(),
                        seqlens=np.array([64, 200], dtype=np.int32), s_q=1, h_q=16, h_kv=1,
                        causal=False, scale=float(D ** -0.5), meta={"seed": seed, "pool_pages": 8})
    if name == "membound":
        return make_workload(np.full(32, 4096), s_q=1, h_q=16, seed=seed, name=name, **kw)
    if name == "mtp":
        rng = np.random.default_rng(1000 + seed)
        lens = rng.integers(1024, 8193, size=64)
        return make_workload(lens, s_q=2, h_q=128, causal=True, seed=seed, name=name, **kw)
    if name == "large":
        return make_workload(np.full(128, 4096), s_q=1, h_q=128, seed=seed, name=name, **kw)
    if name == "ragged":
        rng = np.random.default_rng(1000 + seed)
        lens = np.clip(np.rint(rng.lognormal(np.log(2048.0), 1.0, size=16)), 1, 32768)
        lens[0] = 32768
        lens[8] = 32768
        return make_workload(lens.astype(np.int32), s_q=1, h_q=64, seed=seed, name=name, **kw)
    if name == "hkv2":  # two latent KV heads, 16 query heads each
        return make_workload(np.full(32, 4096), s_q=1, h_q=32, h_kv=2, seed=seed, name=name, **kw)
    raise KeyError(name)

