"""mla_decode_noalloc (the entry point without a workspace argument, for
callers that cannot allocate device memory) against mla_decode on the same
inputs, through the C ABI: two calls in a row, the second with a smaller
input, and a call too large for the library's scratch."""
import numpy as np
import pytest

import oracle
from mla_decode_attention_split_amd import synth
from parity import bf16_bits_of, check_parity, log, to_device

pytestmark = pytest.mark.gpu


def _both(w):
    import torch
    import mla_decode_attention_split_amd as mla
    q, kv, bt, sl = to_device(w)
    meta, splits = mla.mla_get_metadata(sl, w.rows_per_kv_head, w.h_kv)
    out_n = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=q.dtype, device=q.device)
    lse_n = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=q.device)
    mla.mla_decode_noalloc(q, kv, bt, sl, meta, splits, causal=w.causal, softmax_scale=w.scale,
                           out=out_n, lse=lse_n)
    out_r, lse_r = mla.mla_decode(q, kv, bt, sl, meta, splits, causal=w.causal, softmax_scale=w.scale)
    torch.cuda.synchronize()
    return out_n, lse_n, out_r, lse_r


def test_noalloc_matches_decode_twice():
    import torch
    assert torch.cuda.is_available(), "needs an MI355X"
    first = synth.named_workload("mtp")  # ~101 MB of split partials, below the 128 MiB scratch
    second = synth.make_workload([3000, 17, 0, 900, 4096, 65], s_q=1, h_q=16, seed=99)
    for w, what in ((first, "mtp (first call)"), (second, "small batch (second call)")):
        log(f"[case] noalloc {what}: B={w.batch} s_q={w.s_q} h_q={w.h_q}")
        out_n, lse_n, out_r, lse_r = _both(w)
        np.testing.assert_array_equal(bf16_bits_of(out_n), bf16_bits_of(out_r))
        np.testing.assert_array_equal(lse_n.cpu().numpy(), lse_r.cpu().numpy())
        if w is second:
            check_parity(out_n.float().cpu().numpy().astype(np.float64),
                         lse_n.cpu().numpy().astype(np.float64),
                         *oracle.decode(w.q, w.kcache, w.block_table, w.seqlens, causal=w.causal,
                                        scale=w.scale), what="noalloc small batch")


def test_noalloc_rejects_oversized_call():
    import torch
    import mla_decode_attention_split_amd as mla
    w = synth.make_workload([100, 200], s_q=2, h_q=128, causal=True, seed=98)
    q, kv, bt, sl = to_device(w)
    # 8192 parts x 256 rows x 2052 B of partials is far beyond the scratch
    meta, splits = mla.mla_get_metadata(sl, w.rows_per_kv_head, 1, num_parts=8192)
    log("[case] noalloc oversized: 8192 parts, 256 rows per KV head")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_noalloc(q, kv, bt, sl, meta, splits, causal=True, softmax_scale=w.scale)
    assert e.value.status == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
