"""Helpers shared by the GPU parity tests: upload a synthetic workload, run
the HIP path through the C ABI binding, and compare with the oracle.

Acceptance (the tolerance of the benchmark spec for this path):
  out (bf16 vs the fp64 oracle): max |diff| <= 2e-2 and
      ||diff||_F / ||ref||_F <= 5e-3 over the whole tensor;
  lse (fp32): max |diff| <= 1e-3 on rows with a visible key;
  rows without a visible key: out exactly 0 and lse exactly -inf.
"""
from __future__ import annotations

import sys

import numpy as np

OUT_MAX_ABS = 2e-2
OUT_REL_FRO = 5e-3
LSE_MAX_ABS = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(w, device="cuda"):
    import torch
    t = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    q = torch.from_numpy(w.q.view(np.int16)).to(device).view(t)
    kv = torch.from_numpy(w.kcache.view(np.int16)).to(device).view(t)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table, dtype=np.int32)).to(device)
    sl = torch.from_numpy(np.ascontiguousarray(w.seqlens, dtype=np.int32)).to(device)
    return q, kv, bt, sl


def run_gpu(w, *, num_parts=None, fixed_cost=None, tensors=None, return_meta=False):
    import torch
    import mla_decode_attention_split_amd as mla
    q, kv, bt, sl = tensors if tensors is not None else to_device(w)
    meta, splits = mla.mla_get_metadata(sl, w.rows_per_kv_head, w.h_kv, num_parts=num_parts,
                                        fixed_cost=fixed_cost)
    out, lse = mla.mla_decode(q, kv, bt, sl, meta, splits, causal=w.causal,
                              softmax_scale=w.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if return_meta:
        return o, l, meta.cpu().numpy(), splits.cpu().numpy()
    return o, l


def bf16_bits_of(out_t):
    """Raw bf16 bits of a device tensor (for bitwise comparisons)."""
    import torch
    return out_t.view(torch.int16).cpu().numpy()


def check_parity(out, lse, ref_out, ref_lse, what=""):
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: empty-row pattern differs"
    assert np.all(np.isneginf(lse[~fin])), f"{what}: empty rows must have lse -inf"
    assert np.all(out[~fin] == 0), f"{what}: empty rows must have out 0"
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    diff = out - ref_out
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    ref_norm = float(np.linalg.norm(ref_out))
    rel = float(np.linalg.norm(diff) / ref_norm) if ref_norm > 0 else 0.0
    lse_err = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    log(f"  {what}: out max|d| {max_abs:.3e} rel_fro {rel:.3e}  lse max|d| {lse_err:.3e}")
    assert max_abs <= OUT_MAX_ABS, f"{what}: out max abs {max_abs}"
    assert rel <= OUT_REL_FRO, f"{what}: out rel fro {rel}"
    assert lse_err <= LSE_MAX_ABS, f"{what}: lse max abs {lse_err}"
    return max_abs, rel, lse_err


def subset(w, seqs):
    """The same workload restricted to some sequences (pages shared)."""
    from mla_decode_attention_split_amd.synth import Workload
    seqs = np.asarray(seqs)
    return Workload(name=w.name + "-subset", q=np.ascontiguousarray(w.q[seqs]), kcache=w.kcache,
                    block_table=np.ascontiguousarray(w.block_table[seqs]),
                    seqlens=np.ascontiguousarray(w.seqlens[seqs]), s_q=w.s_q, h_q=w.h_q,
                    h_kv=w.h_kv, causal=w.causal, scale=w.scale, meta=dict(w.meta), dtype=w.dtype)
