"""GPU parity: the HIP path (through the C ABI binding) against the CPU oracle.

Every case prints its name and shape before touching the GPU.  Tolerances
are in tests/parity.py.
"""
import numpy as np
import pytest

import oracle
from mla_decode_attention_split_amd import synth
from parity import bf16_bits_of, check_parity, log, run_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    import mla_decode_attention_split_amd as mla
    mla._load()  # raises if the HIP library is missing


def ref(w):
    return oracle.decode(w.q, w.kcache, w.block_table, w.seqlens, causal=w.causal, scale=w.scale,
                         dtype=w.dtype)


def case(w, what):
    log(f"[case] {what}: B={w.batch} s_q={w.s_q} h_q={w.h_q} h_kv={w.h_kv} causal={w.causal} "
        f"N={list(map(int, w.seqlens))[:8]}{'...' if w.batch > 8 else ''}")


def test_tiny_workload():
    w = synth.named_workload("tiny")
    case(w, "tiny")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what="tiny")


@pytest.mark.parametrize("seed", range(16))
def test_random_small_shapes(seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 6))
    s_q = int(rng.integers(1, 5))
    h_q = int(rng.choice([16, 32, 64, 128]))
    causal = bool(rng.integers(0, 2))
    lens = rng.integers(0, 701, size=B)
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=causal, seed=seed,
                            extra_pages=int(rng.integers(0, 4)))
    case(w, f"random seed {seed}")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"seed {seed}")


@pytest.mark.parametrize("h_q,s_q", [(8, 1), (24, 1), (40, 1), (16, 3), (48, 3), (128, 3),
                                     (96, 1), (16, 8), (64, 8), (128, 8)])
def test_row_tile_boundaries(h_q, s_q):
    w = synth.make_workload([130, 77, 300], s_q=s_q, h_q=h_q, causal=True, seed=h_q + s_q)
    case(w, f"rows {s_q * h_q}")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"M={s_q * h_q}")


@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True), (4, True)])
def test_edge_lengths(s_q, causal):
    lens = [0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 1000]
    w = synth.make_workload(lens, s_q=s_q, h_q=16, causal=causal, seed=40 + s_q)
    case(w, "edge lengths")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"edge s_q={s_q}")


@pytest.mark.parametrize("case_name", ["all_empty", "one", "ones", "leading_empty", "trailing_empty",
                                       "more_parts_than_units", "one_long_many_short"])
def test_metadata_bitexact_edges(case_name):
    """Batches that put part boundaries on empty sequences, leave parts with no
    sequence, or pack many sequences into one part (the per-part search for the
    first and last sequence at its limits)."""
    import mla_decode_attention_split_amd as mla
    import torch
    lens = {
        "all_empty": np.zeros(40, np.int32),
        "one": np.array([5000], np.int32),
        "ones": np.ones(300, np.int32),
        "leading_empty": np.concatenate([np.zeros(100, np.int32), np.full(20, 3000, np.int32)]),
        "trailing_empty": np.concatenate([np.full(20, 3000, np.int32), np.zeros(100, np.int32)]),
        "more_parts_than_units": np.array([31, 0, 33, 1], np.int32),
        "one_long_many_short": np.concatenate([np.array([65536], np.int32),
                                               np.full(500, 7, np.int32)]),
    }[case_name]
    for num_parts, fixed_cost in [(1, 1), (8, 2), (256, 2), (4096, 3)]:
        log(f"[case] metadata edge {case_name}: B={lens.size} parts={num_parts} fixed={fixed_cost}")
        sl = torch.from_numpy(lens).cuda()
        meta, splits = mla.mla_get_metadata(sl, 16, 1, num_parts=num_parts, fixed_cost=fixed_cost)
        torch.cuda.synchronize()
        rmeta, rsplits = oracle.schedule(lens, num_parts=num_parts, fixed_cost=fixed_cost,
                                         unit_tokens=32)
        np.testing.assert_array_equal(meta.cpu().numpy(), rmeta)
        np.testing.assert_array_equal(splits.cpu().numpy(), rsplits)


def test_metadata_shape_tiles():
    """Tile rows, fixed cost and default part count follow the row count: 64-row
    tiles up to 64 rows per KV head, 128-row tiles above with one KV head
    (64-row tiles with several)."""
    import mla_decode_attention_split_amd as mla
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, h_kv, tr in [(16, 1, 16), (32, 1, 32), (64, 1, 64), (65, 1, 128), (256, 1, 128),
                        (128, 2, 64), (256, 4, 64)]:
        parts, words = mla.mla_metadata_shape(32, M, h_kv)
        tile, m_tiles, fixed = mla.mla_tile_shape(M, h_kv)
        assert words == 8
        assert tile == tr, (M, tile)
        assert m_tiles == (M + tr - 1) // tr
        assert fixed == max(3, (tr + 31) // 32 + 1)
        per = cus // (m_tiles * h_kv)
        assert parts == (per // 8 * 8 if per >= 8 else 8), (M, h_kv, parts)
        # the default call (no overrides) uses exactly these parameters
        lens = np.arange(0, 3000, 97, dtype=np.int32)
        sl = torch.from_numpy(lens).cuda()
        meta, splits = mla.mla_get_metadata(sl, M, h_kv)
        torch.cuda.synchronize()
        rmeta, rsplits = oracle.schedule(lens, num_parts=parts, fixed_cost=fixed, unit_tokens=32)
        np.testing.assert_array_equal(meta.cpu().numpy(), rmeta)
        np.testing.assert_array_equal(splits.cpu().numpy(), rsplits)


def test_metadata_bitexact():
    import mla_decode_attention_split_amd as mla
    rng = np.random.default_rng(7)
    import torch
    # the last three trials take the scheduler's other two batch/part regimes
    # (more than 1024 sequences; more than 4096 parts) and the largest batch
    special = [(2000, 256), (500, 5000), (16384, 256)]
    for trial in range(12 + len(special)):
        if trial < 12:
            B = int(rng.integers(1, 300))
            num_parts = int(rng.choice([1, 7, 8, 64, 128, 256, 1000]))
        else:
            B, num_parts = special[trial - 12]
        lens = rng.integers(0, 20000 if B < 1000 else 3000, size=B).astype(np.int32)
        if trial % 3 == 0:
            lens[rng.integers(0, B, size=max(1, B // 5))] = 0
        fixed_cost = int(rng.integers(1, 8))
        log(f"[case] metadata trial {trial}: B={B} parts={num_parts} fixed={fixed_cost}")
        sl = torch.from_numpy(lens).cuda()
        meta, splits = mla.mla_get_metadata(sl, 16, 1, num_parts=num_parts, fixed_cost=fixed_cost)
        torch.cuda.synchronize()
        rmeta, rsplits = oracle.schedule(lens, num_parts=num_parts, fixed_cost=fixed_cost,
                                         unit_tokens=32)
        np.testing.assert_array_equal(meta.cpu().numpy(), rmeta)
        np.testing.assert_array_equal(splits.cpu().numpy(), rsplits)


def test_metadata_even_halves():
    """Equal sequences over twice as many parts: the device scheduler cuts each
    one exactly in half (one piece per part), as the oracle's rule does."""
    import mla_decode_attention_split_amd as mla
    import torch
    log("[case] metadata even halves: B=128 N=4096 parts=256 fixed=5")
    lens = np.full(128, 4096, dtype=np.int32)
    meta, splits = mla.mla_get_metadata(torch.from_numpy(lens).cuda(), 128, 1, num_parts=256,
                                        fixed_cost=5)
    torch.cuda.synchronize()
    rmeta, rsplits = oracle.schedule(lens, num_parts=256, fixed_cost=5, unit_tokens=32)
    np.testing.assert_array_equal(meta.cpu().numpy(), rmeta)
    np.testing.assert_array_equal(splits.cpu().numpy(), rsplits)
    np.testing.assert_array_equal(rsplits, np.arange(0, 257, 2))


@pytest.mark.parametrize("num_parts", [1, 7, 64, None])
def test_split_count_does_not_change_result(num_parts):
    lens = [5000, 33, 1, 700, 64, 2048, 0, 3000]
    w = synth.make_workload(lens, s_q=2, h_q=64, causal=True, seed=21)
    case(w, f"num_parts={num_parts}")
    out, lse = run_gpu(w, num_parts=num_parts)
    check_parity(out, lse, *ref(w), what=f"parts={num_parts}")


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (32, 1), (64, 1), (16, 8)])
@pytest.mark.parametrize("num_parts", [3, 8])
def test_many_pieces_per_part(h_q, s_q, num_parts):
    """Parts that hold many short sequences, some empty, for every tile shape:
    the piece epilogues (the first non-last piece's output held back to the
    end of the part in 16-row tiles, the others written at once)."""
    rng = np.random.default_rng(60 + h_q + s_q + num_parts)
    lens = rng.integers(1, 400, size=30)
    lens[[3, 11, 12, 25]] = 0
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=s_q > 1, seed=61 + num_parts)
    case(w, f"many pieces per part, parts={num_parts}")
    out, lse = run_gpu(w, num_parts=num_parts)
    check_parity(out, lse, *ref(w), what=f"h_q={h_q} s_q={s_q} parts={num_parts}")


@pytest.mark.parametrize("lens,num_parts,h_q,s_q", [([10000], 17, 16, 1), ([10000], 100, 16, 1),
                                                     ([20000, 50], 129, 32, 2), ([3000, 9000, 1], 160, 16, 3)])
def test_combine_many_pieces(lens, num_parts, h_q, s_q):
    """Sequences split into many pieces: the combine's shared-row layout (four
    waves per row, 16-aligned piece ranges, some of them empty, ranges past
    the first 64 pieces) against the oracle."""
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=s_q > 1, seed=31 + num_parts)
    case(w, f"many pieces parts={num_parts}")
    out, lse, _, splits = run_gpu(w, num_parts=num_parts, return_meta=True)
    assert np.diff(splits).max() > 16  # the shared-row layout is taken
    check_parity(out, lse, *ref(w), what=f"parts={num_parts}")


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (32, 1), (64, 1), (128, 1), (64, 2)])
@pytest.mark.parametrize("num_parts", [1, 3])
def test_part_with_more_than_64_pieces(h_q, s_q, num_parts):
    """A part holding hundreds of pieces (300 short sequences, some empty): the
    kernel's page list cannot hold them, so lengths past the 64th piece and
    every page index are read one by one while streaming."""
    rng = np.random.default_rng(80 + h_q + s_q + num_parts)
    lens = rng.integers(0, 101, size=300)
    lens[rng.integers(0, 300, size=30)] = 0
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=s_q > 1, seed=81 + num_parts)
    case(w, f"more than 64 pieces per part, parts={num_parts}")
    out, lse, meta, _ = run_gpu(w, num_parts=num_parts, return_meta=True)
    pieces = meta[:, 2] - meta[:, 0] + 1
    assert pieces.max() > 64, pieces.max()
    check_parity(out, lse, *ref(w), what=f"h_q={h_q} s_q={s_q} parts={num_parts}")


@pytest.mark.parametrize("B,num_parts,h_q", [(2000, None, 16), (1500, 300, 128), (600, 5000, 16)])
def test_large_batches(B, num_parts, h_q):
    """Batches past the scheduler's fast variant (more than 1024 sequences, or
    more than 4096 parts), decoded end to end."""
    rng = np.random.default_rng(90 + B)
    lens = rng.integers(0, 300, size=B)
    w = synth.make_workload(lens, s_q=1, h_q=h_q, seed=91 + B)
    case(w, f"large batch B={B} parts={num_parts}")
    out, lse = run_gpu(w, num_parts=num_parts)
    check_parity(out, lse, *ref(w), what=f"B={B} parts={num_parts}")


@pytest.mark.parametrize("lens,h_q,s_q", [([4096] * 8, 16, 1), (list(range(100, 4100, 100)), 16, 1),
                                          ([3000, 1, 0, 7000, 2500], 128, 2), ([4096] * 12, 32, 2)])
def test_splitkv_then_combine(lens, h_q, s_q):
    """The benchmark's timed path: the metadata call, then the main kernel alone
    (mla_decode_splitkv), then the combine alone (mla_decode_combine), through
    the binding.  Bitwise equal to mla_decode, and within tolerance of the
    oracle; the cases take both combine layouts (many or few pieces per
    sequence)."""
    import torch
    import mla_decode_attention_split_amd as mla
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=s_q > 1, seed=95 + len(lens))
    case(w, "split then combine")
    q, kv, bt, sl = to_device(w)
    meta, splits = mla.mla_get_metadata(sl, w.rows_per_kv_head, w.h_kv)
    out, lse, ws = mla.mla_decode_splitkv(q, kv, bt, sl, meta, splits, causal=w.causal,
                                          softmax_scale=w.scale)
    mla.mla_decode_combine(splits, out, lse, ws, num_parts=meta.shape[0], h_kv=w.h_kv)
    o2, l2 = mla.mla_decode(q, kv, bt, sl, meta, splits, causal=w.causal, softmax_scale=w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits_of(out), bf16_bits_of(o2))
    np.testing.assert_array_equal(lse.cpu().numpy(), l2.cpu().numpy())
    check_parity(out.float().cpu().numpy().astype(np.float64),
                 lse.cpu().numpy().astype(np.float64), *ref(w), what="split then combine")


def test_deterministic_bitwise():
    import torch
    import mla_decode_attention_split_amd as mla
    w = synth.make_workload([4000, 100, 2500], s_q=1, h_q=128, seed=22)
    case(w, "determinism")
    q, kv, bt, sl = to_device(w)
    meta, splits = mla.mla_get_metadata(sl, w.rows_per_kv_head, 1)
    o1, l1 = mla.mla_decode(q, kv, bt, sl, meta, splits, softmax_scale=w.scale)
    o2, l2 = mla.mla_decode(q, kv, bt, sl, meta, splits, softmax_scale=w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits_of(o1), bf16_bits_of(o2))
    np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_page_permutation_bitwise():
    w = synth.make_workload([300, 2000, 65], s_q=2, h_q=32, causal=True, seed=23, extra_pages=5)
    case(w, "page permutation")
    o1, l1 = run_gpu(w)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.kcache.shape[0])
    moved = np.empty_like(w.kcache)
    moved[perm] = w.kcache
    w.kcache = moved
    w.block_table = perm[w.block_table].astype(np.int32)
    o2, l2 = run_gpu(w)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_poison_in_unread_memory():
    lens = [65, 128, 3, 0, 191, 1000]
    clean = synth.make_workload(lens, s_q=2, h_q=16, causal=True, seed=24, extra_pages=2,
                                table_width=20)
    dirty = synth.make_workload(lens, s_q=2, h_q=16, causal=True, seed=24, extra_pages=2,
                                table_width=20, pad="poison", poison_tail=True)
    case(dirty, "poison")
    o1, l1 = run_gpu(clean)
    o2, l2 = run_gpu(dirty)
    assert np.isfinite(o2).all()
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    check_parity(o2, l2, *ref(dirty), what="poison")


def test_two_kv_heads():
    w = synth.make_workload([300, 1200], s_q=2, h_q=32, h_kv=2, causal=True, seed=25)
    case(w, "h_kv=2")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what="h_kv=2")


@pytest.mark.parametrize("h_q,s_q,h_kv", [(128, 2, 2), (64, 3, 2), (128, 4, 4)])
def test_kv_heads_many_rows(h_q, s_q, h_kv):
    """Several KV heads with more than 64 query rows per head (64-row tiles,
    several per head, with per-lane query offsets), including a partial row
    tile."""
    w = synth.make_workload([700, 129, 64], s_q=s_q, h_q=h_q, h_kv=h_kv, causal=True,
                            seed=27 + h_q + s_q)
    case(w, f"h_kv={h_kv} rows {w.rows_per_kv_head}")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"h_kv={h_kv} M={w.rows_per_kv_head}")


@pytest.mark.parametrize("h_q,s_q,h_kv", [(32, 1, 2), (16, 2, 2), (24, 1, 2), (64, 2, 4), (32, 2, 2)])
@pytest.mark.parametrize("num_parts", [1, 5])
def test_kv_heads_small_tiles_many_pieces(h_q, s_q, h_kv, num_parts):
    """Several KV heads with 16- or 32-row tiles, whose query rows are
    loaded straight into registers through per-lane offsets (row m of a KV
    head is token m / hpg, head g hpg + m % hpg), reloaded for every piece:
    parts of many short pieces (some sequences empty), causal when s_q > 1,
    and a partial row tile (24 heads over 2 KV heads: 12 rows per head)."""
    rng = np.random.default_rng(30 + h_q + s_q + h_kv + num_parts)
    lens = rng.integers(0, 300, size=60)
    lens[rng.integers(0, 60, size=6)] = 0
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=s_q > 1,
                            seed=31 + h_q + num_parts)
    case(w, f"h_kv={h_kv} rows {w.rows_per_kv_head}, many pieces, parts={num_parts}")
    out, lse, meta, _ = run_gpu(w, num_parts=num_parts, return_meta=True)
    pieces = meta[:, 2] - meta[:, 0] + 1
    assert pieces.max() > 2, pieces.max()
    check_parity(out, lse, *ref(w), what=f"h_kv={h_kv} M={w.rows_per_kv_head} parts={num_parts}")


def test_pool_past_4gib():
    """Pages at the top of a cache pool larger than 4 GiB (64-bit byte offsets
    of pages): the used pages of a small workload are placed at the pool's
    end, the block table shifted to match; the oracle runs on the compact pool."""
    import torch
    w = synth.make_workload([5000, 3000, 77], s_q=2, h_q=32, causal=True, seed=71)
    q, kv, bt, sl = to_device(w)
    num_pages = 60000  # 60000 x 73,728 B = 4.42 GB
    used = kv.shape[0]
    base = num_pages - used
    assert base * 64 * 1152 > (1 << 32)
    log(f"[case] pool of {num_pages} pages, used pages from index {base}")
    big = torch.zeros((num_pages,) + tuple(kv.shape[1:]), dtype=kv.dtype, device=kv.device)
    big[base:] = kv
    out, lse = run_gpu(w, tensors=(q, big, bt + base, sl))
    del big
    torch.cuda.empty_cache()
    check_parity(out, lse, *ref(w), what="pool past 4 GiB")


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (64, 1), (128, 2)])
def test_table_entry_outside_pool_reads_zeros(h_q, s_q):
    """A block_table entry equal to num_pages reads as a page of zeros.  The
    pool handed to the library is a view of one page fewer than the allocated
    tensor, so the entry still points into allocated memory (filled with 3.0):
    reading it would change the result, not fault.  Reference: the oracle on
    the same table with page num_pages made of zeros.  Covers the 16-row,
    64-row and 128-row tiles."""
    import dataclasses
    import torch
    w = synth.make_workload([300, 200], s_q=s_q, h_q=h_q, causal=s_q > 1, seed=81 + h_q)
    case(w, f"table entry outside the pool, h_q={h_q}")
    q, kv, bt, sl = to_device(w)
    P = kv.shape[0]
    alloc = torch.full((P + 1,) + tuple(kv.shape[1:]), 3.0, dtype=kv.dtype, device=kv.device)
    alloc[:P] = kv
    bt_bad = bt.clone()
    bt_bad[0, 1] = P  # the second page of sequence 0 (keys 64..127 of 300)
    out, lse = run_gpu(w, tensors=(q, alloc[:P], bt_bad, sl))
    zero_page = np.zeros((1,) + w.kcache.shape[1:], dtype=w.kcache.dtype)
    table = w.block_table.copy()
    table[0, 1] = P
    w_ref = dataclasses.replace(w, kcache=np.concatenate([w.kcache, zero_page]), block_table=table)
    check_parity(out, lse, *ref(w_ref), what=f"entry outside the pool, h_q={h_q}")


@pytest.mark.parametrize("lens,s_q,h_q", [([131072], 1, 16), ([65536, 1000], 2, 64)])
def test_long_sequences(lens, s_q, h_q):
    """Sequences of 64K and 128K keys, split over every part of the default
    partition (hundreds of pieces per sequence) and merged by the combine."""
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=s_q > 1, seed=72 + s_q)
    case(w, f"long sequences {lens}")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"long {lens}")


def test_constant_value_rows():
    w = synth.make_workload([500, 37], s_q=1, h_q=16, seed=26)
    c = synth.bf16_bits(np.array([-1.375], dtype=np.float32))[0]
    w.kcache[..., :512] = c
    case(w, "constant V")
    out, lse = run_gpu(w)
    np.testing.assert_array_equal(out, -1.375)
    check_parity(out, lse, *ref(w), what="constant V")


@pytest.mark.parametrize("name", ["membound", "mtp", "large", "ragged", "hkv2"])
def test_full_size(name):
    """Every full-size workload in the benchmark's launch configuration (default
    part count and tile), the whole out and lse tensors against the oracle."""
    w = synth.named_workload(name)
    case(w, f"full {name}")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"{name} (whole output)")


def test_ceiling_helpers_run():
    """The measurement library's probes run on a small pool, including page
    indices outside it (which must load nothing rather than fault)."""
    import torch
    import bench
    log("case: ceiling helpers")
    dev = torch.device("cuda")
    pool = torch.zeros((16, 64 * 576), dtype=torch.bfloat16, device=dev)
    pages = torch.tensor([[0, 5, 15], [3, 16, 1 << 30]], dtype=torch.int32, device=dev)
    isink = torch.zeros(1, dtype=torch.int32, device=dev)
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    bench.ceiling_stream(pool, pages, isink)
    bench.ceiling_mfma(fsink, 8, 10)
    bench.ceiling_mfma(fsink, 8, 11, random_operands=True)
    torch.cuda.synchronize()
    assert int(isink.item()) == 0 and float(fsink.item()) == 0.0


@pytest.mark.parametrize("seed", range(6))
def test_fp16_random_small_shapes(seed):
    """fp16 q and cache (one page lists FP16 beside BF16) against the oracle
    reading the same bits as fp16."""
    rng = np.random.default_rng(700 + seed)
    B = int(rng.integers(1, 5))
    s_q = int(rng.integers(1, 4))
    h_q = int(rng.choice([16, 32, 64, 128]))
    causal = bool(rng.integers(0, 2))
    lens = rng.integers(1, 1500, size=B)
    w = synth.make_workload(lens, s_q=s_q, h_q=h_q, causal=causal, seed=seed, dtype="fp16")
    case(w, f"fp16 seed {seed}")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"fp16 seed {seed}")


@pytest.mark.parametrize("name", ["membound", "mtp", "large", "ragged", "hkv2"])
def test_fp16_full_size(name):
    """The full-size workloads drawn in fp16, whole outputs against the oracle
    reading the same bits as fp16."""
    w = synth.named_workload(name, dtype="fp16")
    case(w, f"full {name} fp16")
    out, lse = run_gpu(w)
    check_parity(out, lse, *ref(w), what=f"{name} fp16 (whole output)")


@pytest.mark.parametrize("name", ["membound", "mtp", "ragged"])
def test_torch_baseline_matches_oracle(name):
    """The plain PyTorch GPU implementation the benchmark times for comparison
    computes the same attention: its whole output is within the tolerance of
    the oracle, so the baseline being timed is a correct one."""
    import bench
    w = synth.named_workload(name)
    case(w, f"torch baseline {name}")
    q, kv, bt, _ = to_device(w)
    _, out, lse = bench.torch_baseline(w, q, kv, bt, steps=1)
    check_parity(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 *ref(w), what=f"torch baseline {name}")
