"""A whole decode step (metadata call, then decode) captured once as a HIP
graph and replayed with new query rows and new sequence lengths.

The path makes no host synchronisation, allocation or memset: the lengths
are read on the device only, so a captured step stays valid when they
change, as in a serving loop that replays one graph per decode step.  Every
replay is compared bit for bit with the same calls made eagerly on the same
inputs (with eager work and synchronisations between the replays), and two
of them with the oracle.
"""
import numpy as np
import pytest

import oracle
from mla_decode_attention_split_amd import synth
from parity import check_parity, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h_q,s_q,noalloc", [(16, 1, False), (64, 1, False), (128, 2, False),
                                             (16, 1, True)])
def test_decode_step_graph_replays(h_q, s_q, noalloc):
    import torch
    import mla_decode_attention_split_amd as mla

    cap = np.array([2500, 900, 3100, 64, 1700, 40], dtype=np.int32)  # table capacity per sequence
    causal = s_q > 1
    w = synth.make_workload(cap, s_q=s_q, h_q=h_q, causal=causal, seed=70 + h_q + s_q)
    B, M = w.batch, w.rows_per_kv_head
    log(f"[case] graph replays: B={B} s_q={s_q} h_q={h_q} noalloc={noalloc}")
    dev = torch.device("cuda:0")
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    sl = torch.from_numpy(cap.copy()).to(dev)
    parts, words = mla.mla_metadata_shape(B, M, 1)
    meta = torch.empty((parts, words), dtype=torch.int32, device=dev)
    splits = torch.empty((B + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    ws = torch.empty((mla.mla_workspace_bytes(B, M, 1, parts),), dtype=torch.uint8, device=dev)

    def step():
        mla.mla_get_metadata(sl, M, 1, tile_metadata=meta, num_splits=splits)
        if noalloc:
            mla.mla_decode_noalloc(q, kv, bt, sl, meta, splits, causal=causal, softmax_scale=w.scale,
                                   out=out, lse=lse)
        else:
            mla.mla_decode(q, kv, bt, sl, meta, splits, causal=causal, softmax_scale=w.scale,
                           out=out, lse=lse, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        step()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    rng = np.random.default_rng(71 + h_q)
    for r in range(4):
        lens = (rng.random(B) * (cap + 1)).astype(np.int32)
        if r == 1:
            lens[2] = 0  # an empty sequence
        if r == 3:
            lens = cap.copy()
        q_bits = synth.bf16_bits(rng.standard_normal(w.q.shape).astype(np.float32))
        sl.copy_(torch.from_numpy(lens))
        q.copy_(torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        o_graph, l_graph = out.clone(), lse.clone()
        meta_e, splits_e = mla.mla_get_metadata(sl, M, 1)
        o_eager, l_eager = mla.mla_decode(q, kv, bt, sl, meta_e, splits_e, causal=causal,
                                          softmax_scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_graph.view(torch.int16), o_eager.view(torch.int16)), f"replay {r}: out"
        assert torch.equal(l_graph.view(torch.int32), l_eager.view(torch.int32)), f"replay {r}: lse"
        if r in (1, 3):
            ref_out, ref_lse = oracle.decode(q_bits, w.kcache, w.block_table, lens, causal=causal,
                                             scale=w.scale)
            check_parity(o_graph.float().cpu().numpy().astype(np.float64),
                         l_graph.cpu().numpy().astype(np.float64), ref_out, ref_lse,
                         what=f"graph replay {r}")
