"""Pins of the CPU oracle to things other than itself (CPU only).

Each check is chosen so that a plausible slip in the oracle -- a dropped rope
term, a wrong page/slot index, a transposed operand, a wrong scale, an
off-by-one causal boundary, a log base, a merge weight -- fails at least one:

* dense float64 brute force on unpaged K/V (numpy + scipy.special.logsumexp);
* a library routine on special cases: torch's scaled_dot_product_attention
  (float64, CPU) with V = K[:, :512] and a bottom-right causal mask;
* closed forms: constant V, q = 0, one key, two keys;
* invariants: page permutation, split independence, lse recomputes the
  softmax denominator, the causal boundary, rope dims only act through the
  scores, poison in unread memory, KV-head grouping;
* the scheduler against brute-force enumeration of every page's part and the
  exact-cover property.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from mla_decode_attention_split_amd import synth
from mla_decode_attention_split_amd.synth import D, DV, PAGE, bf16_bits, bf16_to_f32

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def run_oracle(w, **kw):
    return oracle.decode(w.q, w.kcache, w.block_table, w.seqlens, causal=w.causal, scale=w.scale,
                         dtype=w.dtype, **kw)


def to64(bits, dtype):
    """16-bit bit patterns -> float64 by numpy's own conversions."""
    if dtype == "fp16":
        return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return bf16_to_f32(bits).astype(np.float64)


def dense_keys(w, b):
    """[N_b, h_kv, 576] float64 keys of sequence b, gathered with numpy fancy indexing."""
    kc = to64(w.kcache, w.dtype)
    n = int(w.seqlens[b])
    j = np.arange(n)
    return kc[w.block_table[b, j // PAGE], j % PAGE]


def visible(n, s_q, t, causal):
    return max(0, min(n, n - s_q + t + 1) if causal else n)


def dense_reference(w):
    """Brute force: unpaged K/V, full score matrix, masked logsumexp."""
    q = to64(w.q, w.dtype)
    B, s_q, h_q, _ = q.shape
    hpg = h_q // w.h_kv
    out = np.zeros((B, s_q, h_q, DV))
    lse = np.full((B, s_q, h_q), -np.inf)
    for b in range(B):
        K = dense_keys(w, b)
        n = K.shape[0]
        for g in range(w.h_kv):
            Kg = K[:, g, :]
            Vg = Kg[:, :DV]
            Qg = q[b, :, g * hpg:(g + 1) * hpg, :]          # [s_q, hpg, 576]
            S = (Qg @ Kg.T) * w.scale                        # [s_q, hpg, n]
            vis = np.array([visible(n, s_q, t, w.causal) for t in range(s_q)])
            mask = np.arange(n)[None, :] < vis[:, None]      # [s_q, n]
            Sm = np.where(mask[:, None, :], S, -np.inf)
            L = scipy.special.logsumexp(Sm, axis=-1)         # [s_q, hpg]
            P = np.where(mask[:, None, :], np.exp(Sm - np.where(np.isfinite(L), L, 0)[..., None]),
                         0.0)
            out[b, :, g * hpg:(g + 1) * hpg, :] = P @ Vg
            lse[b, :, g * hpg:(g + 1) * hpg] = L
    return out, lse


def random_tiny(seed, dtype="bf16"):
    rng = np.random.default_rng(10_000 + seed)
    B = int(rng.integers(1, 4))
    s_q = int(rng.integers(1, 5))
    h_kv = int(rng.choice([1, 1, 2]))
    h_q = int(rng.choice([16, 32])) if h_kv == 1 else 16
    causal = bool(rng.integers(0, 2))
    lens = rng.integers(0, 301, size=B)
    if seed % 5 == 0:
        lens[0] = int(rng.integers(0, 4))          # empty / causal-empty rows
    return synth.make_workload(lens, s_q=s_q, h_q=h_q, h_kv=h_kv, causal=causal, seed=seed,
                               extra_pages=int(rng.integers(0, 3)), dtype=dtype)


def assert_close(a, b, rtol=1e-11, atol=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    np.testing.assert_allclose(a[fin], b[fin], rtol=rtol, atol=atol)


# --------------------------------------------------------------------------
# Whole definition: dense brute force and a library routine
# --------------------------------------------------------------------------

def test_tiny_named_workload_matches_dense():
    w = synth.named_workload("tiny")
    out, lse = run_oracle(w)
    rout, rlse = dense_reference(w)
    assert_close(out, rout)
    assert_close(lse, rlse)


@pytest.mark.parametrize("seed", range(60))
def test_random_tiny_matches_dense(seed):
    w = random_tiny(seed)
    out, lse = run_oracle(w)
    rout, rlse = dense_reference(w)
    assert_close(out, rout)
    assert_close(lse, rlse)


@pytest.mark.parametrize("causal,s_q", [(False, 1), (True, 3), (False, 2)])
def test_matches_torch_sdpa_float64(causal, s_q):
    w = synth.make_workload([37, 130, 64], s_q=s_q, h_q=16, causal=causal, seed=7)
    out, lse = run_oracle(w)
    q = torch.from_numpy(bf16_to_f32(w.q).astype(np.float64))
    for b in range(w.batch):
        K = torch.from_numpy(dense_keys(w, b)[:, 0, :])      # [n, 576]
        V = K[:, :DV].contiguous()
        n = K.shape[0]
        qb = q[b].permute(1, 0, 2).contiguous()               # [h_q, s_q, 576]
        mask = torch.ones(s_q, n, dtype=torch.bool)
        if causal:
            mask = torch.ones(s_q, n, dtype=torch.bool).tril(diagonal=n - s_q)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qb, K.expand(16, n, D), V.expand(16, n, DV), attn_mask=mask, scale=w.scale)
        scores = (qb @ K.T) * w.scale
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[b], ref_lse.T.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def test_constant_v_gives_that_constant():
    w = synth.make_workload([1, 77, 200], s_q=2, h_q=16, causal=True, seed=3)
    c = bf16_bits(np.array([0.71875], dtype=np.float32))[0]
    w.kcache[..., :DV] = c
    out, lse = run_oracle(w)
    for b, n in enumerate(w.seqlens):
        for t in range(w.s_q):
            if visible(int(n), w.s_q, t, True) == 0:      # N=1, s_q=2: row 0 sees nothing
                assert (out[b, t] == 0).all() and np.isneginf(lse[b, t]).all()
            else:
                np.testing.assert_allclose(out[b, t], 0.71875, rtol=1e-14, atol=0)


def test_zero_query_gives_log_count_and_mean():
    w = synth.make_workload([5, 64, 129], s_q=3, h_q=16, causal=True, seed=4)
    w.q[...] = 0
    out, lse = run_oracle(w)
    for b in range(w.batch):
        K = dense_keys(w, b)[:, 0, :DV]
        n = K.shape[0]
        for t in range(w.s_q):
            L = visible(n, w.s_q, t, True)
            np.testing.assert_allclose(lse[b, t], math.log(L), rtol=1e-14)
            np.testing.assert_allclose(out[b, t], np.broadcast_to(K[:L].mean(0), (16, DV)),
                                       rtol=1e-12, atol=1e-14)


def test_single_key_returns_its_value_row():
    w = synth.make_workload([1, 1], s_q=1, h_q=16, seed=5)
    out, lse = run_oracle(w)
    q = bf16_to_f32(w.q).astype(np.float64)
    for b in range(2):
        k = dense_keys(w, b)[0, 0]
        np.testing.assert_array_equal(out[b, 0], np.broadcast_to(k[:DV], (16, DV)))
        s0 = np.array([math.fsum(q[b, 0, h] * k) for h in range(16)]) * w.scale
        np.testing.assert_allclose(lse[b, 0], s0, rtol=1e-13, atol=1e-14)


def test_two_keys_closed_form():
    # q = 24 * e_0, key0[0] = 0, key1[0] = 1 and scale 1/24: scores are exactly 0 and 1.
    w = synth.make_workload([2], s_q=1, h_q=16, seed=6, scale=1.0 / 24.0)
    w.q[...] = 0
    w.q[..., 0] = bf16_bits(np.array([24.0], dtype=np.float32))[0]
    p0 = w.block_table[0, 0]
    w.kcache[p0, 0, 0, 0] = bf16_bits(np.array([0.0], dtype=np.float32))[0]
    w.kcache[p0, 1, 0, 0] = bf16_bits(np.array([1.0], dtype=np.float32))[0]
    out, lse = run_oracle(w)
    v0 = bf16_to_f32(w.kcache[p0, 0, 0, :DV]).astype(np.float64)
    v1 = bf16_to_f32(w.kcache[p0, 1, 0, :DV]).astype(np.float64)
    e = math.e
    np.testing.assert_allclose(lse[0, 0], math.log(1.0 + e), rtol=1e-15)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v0 / (1 + e) + v1 * e / (1 + e),
                                                          (16, DV)), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def test_page_permutation_is_bitwise_invariant():
    w = synth.make_workload([64, 200, 1, 333], s_q=2, h_q=16, causal=True, seed=8, extra_pages=3)
    out, lse = run_oracle(w)
    rng = np.random.default_rng(99)
    P = w.kcache.shape[0]
    perm = rng.permutation(P)                 # new position of old page i is perm[i]
    moved = np.empty_like(w.kcache)
    moved[perm] = w.kcache
    table = perm[w.block_table].astype(np.int32)
    out2, lse2 = oracle.decode(w.q, moved, table, w.seqlens, causal=True, scale=w.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("seed", range(8))
def test_split_pieces_merge_to_unsplit(seed):
    w = random_tiny(seed)
    out, lse = run_oracle(w)
    rng = np.random.default_rng(seed)
    cuts = []
    for n in w.seqlens:
        k = int(rng.integers(0, 6))
        c = np.unique(rng.integers(1, max(2, int(n)), size=k)) if n > 1 else np.array([], int)
        cuts.append(c[(c > 0) & (c < n)])
    out2, lse2 = oracle.decode_split(w.q, w.kcache, w.block_table, w.seqlens, cuts,
                                     causal=w.causal, scale=w.scale)
    assert_close(out2, out, rtol=1e-12, atol=1e-13)
    assert_close(lse2, lse, rtol=1e-13, atol=1e-13)


def test_lse_is_the_softmax_denominator():
    w = synth.make_workload([300, 17], s_q=2, h_q=16, causal=True, seed=9)
    _, lse = run_oracle(w)
    q = bf16_to_f32(w.q).astype(np.float64)
    for b in range(2):
        K = dense_keys(w, b)[:, 0, :]
        for t in range(2):
            L = visible(K.shape[0], 2, t, True)
            s = (q[b, t] @ K[:L].T) * w.scale
            np.testing.assert_allclose(np.exp(s - lse[b, t][:, None]).sum(-1), 1.0, rtol=1e-12)


def test_causal_boundary():
    n, s_q = 150, 4
    w = synth.make_workload([n], s_q=s_q, h_q=16, causal=True, seed=10)
    out, lse = run_oracle(w)
    for t in range(s_q):
        last_visible = n - s_q + t
        for j, should_change in ((last_visible, True), (last_visible + 1, False)):
            if j >= n:
                continue
            w2 = synth.make_workload([n], s_q=s_q, h_q=16, causal=True, seed=10)
            w2.kcache[w2.block_table[0, j // PAGE], j % PAGE] = bf16_bits(
                np.full(D, 0.5, dtype=np.float32))
            o2, l2 = run_oracle(w2)
            changed = not (np.array_equal(o2[0, t], out[0, t]) and np.array_equal(l2[0, t],
                                                                                  lse[0, t]))
            assert changed == should_change, (t, j)
    # causal with one query token is the same as non-causal
    w1 = synth.make_workload([n, 3], s_q=1, h_q=16, causal=True, seed=11)
    o_c, l_c = run_oracle(w1)
    o_n, l_n = oracle.decode(w1.q, w1.kcache, w1.block_table, w1.seqlens, causal=False,
                             scale=w1.scale)
    np.testing.assert_array_equal(o_c, o_n)
    np.testing.assert_array_equal(l_c, l_n)


def test_rope_dims_act_only_through_scores():
    w = synth.make_workload([90, 140], s_q=1, h_q=16, seed=12)
    rng = np.random.default_rng(0)
    noise = bf16_bits(rng.standard_normal(w.kcache[..., DV:].shape, dtype=np.float32))
    # with the query's rope part zero, the cache's rope part cannot matter
    w.q[..., DV:] = 0
    o1, l1 = run_oracle(w)
    w.kcache[..., DV:] = noise
    o2, l2 = run_oracle(w)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # with a non-zero query rope part it must matter
    w.q[..., DV:] = bf16_bits(np.full(D - DV, 0.25, dtype=np.float32))
    o3, _ = run_oracle(w)
    assert not np.array_equal(o3, o2)


def test_poison_in_unread_memory_is_ignored():
    lens = [65, 128, 3, 0, 191]
    clean = synth.make_workload(lens, s_q=2, h_q=16, causal=True, seed=13, extra_pages=2,
                                table_width=5)
    dirty = synth.make_workload(lens, s_q=2, h_q=16, causal=True, seed=13, extra_pages=2,
                                table_width=5, pad="minus1", poison_tail=True)
    o1, l1 = run_oracle(clean)
    o2, l2 = run_oracle(dirty)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert np.isfinite(o2).all()
    # empty sequence and causally empty rows: out 0, lse -inf
    assert (o2[3] == 0).all() and np.isneginf(l2[3]).all()


def test_kv_head_grouping():
    w = synth.make_workload([70, 129], s_q=2, h_q=16, h_kv=2, causal=False, seed=14)
    out, lse = run_oracle(w)
    # swapping the two KV heads' data swaps the two halves of the query heads
    w_sw = synth.make_workload([70, 129], s_q=2, h_q=16, h_kv=2, causal=False, seed=14)
    w_sw.kcache = np.ascontiguousarray(w_sw.kcache[:, :, ::-1, :])
    w_sw.q = np.ascontiguousarray(np.concatenate([w.q[:, :, 8:], w.q[:, :, :8]], axis=2))
    o2, l2 = run_oracle(w_sw)
    np.testing.assert_array_equal(o2[:, :, :8], out[:, :, 8:])
    np.testing.assert_array_equal(l2[:, :, 8:], lse[:, :, :8])
    # identical KV heads give the single-head result
    w1 = synth.make_workload([70, 129], s_q=2, h_q=16, h_kv=1, seed=15)
    w2 = synth.make_workload([70, 129], s_q=2, h_q=16, h_kv=2, seed=15)
    w2.kcache = np.ascontiguousarray(np.repeat(w1.kcache, 2, axis=2))
    w2.q = w1.q
    w2.block_table = w1.block_table
    o1, l1 = run_oracle(w1)
    o2, l2 = run_oracle(w2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_bad_page_index_is_rejected():
    w = synth.make_workload([70], s_q=1, h_q=16, seed=16)
    w.block_table[0, 1] = w.kcache.shape[0]
    with pytest.raises(ValueError):
        run_oracle(w)


# --------------------------------------------------------------------------
# Scheduler: brute-force enumeration and exact cover
# --------------------------------------------------------------------------

def enumerate_parts(seqlens, num_parts, fixed_cost, unit):
    """Part of every unit, unit by unit, straight from the cost-interval rule:
    a line in half units, each sequence's fixed cost split over its two ends,
    each unit at its midpoint, the line shared evenly by the parts (position
    x in part floor(x num_parts / total), or floor(x / 2) when the line is
    shorter than two positions per part).  Also returns T, the most
    positions any part spans."""
    units = [(int(n) + unit - 1) // unit for n in seqlens]
    total = sum(2 * u + 2 * fixed_cost for u in units)
    span2 = total < 2 * num_parts

    def part(x):
        return x // 2 if span2 else x * num_parts // total

    T = 2 if span2 else -(-total // num_parts)
    pos = 0
    where = []
    for u in units:
        if u == 0:
            where.append([part(pos + fixed_cost)])
        else:
            where.append([part(pos + fixed_cost + 2 * i + 1) for i in range(u)])
        pos += 2 * u + 2 * fixed_cost
    return units, where, T


def pieces_from_meta(meta, seqlens, ns):
    """Expand tile metadata into {(b, split): (part, key_lo, key_hi)}."""
    got = {}
    for p, w in enumerate(meta):
        bb, kb, be, ke, slot0, n_first, n_last, slot_last = (int(x) for x in w)
        if bb > be:
            assert (bb, kb, be, ke) == (0, 0, -1, 0) and (w[4:] == 0).all()
            continue
        k0 = slot0 - int(ns[bb])
        assert n_first == seqlens[bb] and n_last == seqlens[be] and slot_last == ns[be]
        for b in range(bb, be + 1):
            lo = kb if b == bb else 0
            hi = ke if b == be else int(seqlens[b])
            k = k0 if b == bb else 0
            assert (b, k) not in got
            got[(b, k)] = (p, lo, hi)
    return got


@pytest.mark.parametrize("seed", range(40))
def test_schedule_matches_unit_enumeration(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 3000, size=B)
    if seed % 3 == 0:
        lens[rng.integers(0, B)] = 0
    num_parts = int(rng.integers(1, 300))
    fixed_cost = int(rng.integers(1, 6))
    unit = int(rng.choice([16, 32, 64]))
    meta, ns = oracle.schedule(lens, num_parts=num_parts, fixed_cost=fixed_cost, unit_tokens=unit)
    units, where, T = enumerate_parts(lens, num_parts, fixed_cost, unit)
    got = pieces_from_meta(meta, lens, ns)
    assert ns[0] == 0
    for b in range(B):
        parts = sorted(set(where[b]))
        assert parts == list(range(parts[0], parts[-1] + 1))
        assert ns[b + 1] - ns[b] == len(parts)
        covered = []
        for k, part in enumerate(parts):
            p, lo, hi = got[(b, k)]
            assert p == part
            assert lo % unit == 0 and (hi % unit == 0 or hi == lens[b])
            covered.extend(range(lo, hi))
            assert all(where[b][i // unit] == p for i in range(lo, hi))
        assert covered == list(range(int(lens[b])))     # exact cover of the keys, in order
    assert len(got) == ns[-1]
    # balance: no part holds more units of keys than fit in T half units
    per_part = np.zeros(num_parts, dtype=np.int64)
    for (b, k), (p, lo, hi) in got.items():
        per_part[p] += -(-(hi - lo) // unit)
    assert per_part.max() <= (T + 1) // 2


@pytest.mark.parametrize("lens,num_parts,fixed_cost", [([32, 0, 64, 100], 256, 1),
                                                        ([1], 1000, 1), ([0, 0, 5000], 64, 3)])
def test_schedule_tiny_total(lens, num_parts, fixed_cost):
    """Far more parts than cost positions (every part spans 2 half units): every
    sequence's pieces still sit in consecutive parts and cover its keys once."""
    lens = np.asarray(lens)
    meta, ns = oracle.schedule(lens, num_parts=num_parts, fixed_cost=fixed_cost, unit_tokens=32)
    units, where, T = enumerate_parts(lens, num_parts, fixed_cost, 32)
    assert T == 2 or sum(2 * u + 2 * fixed_cost for u in units) > 2 * num_parts
    got = pieces_from_meta(meta, lens, ns)
    for b in range(len(lens)):
        parts = sorted(set(where[b]))
        assert parts == list(range(parts[0], parts[-1] + 1))
        keys = []
        for k in range(ns[b + 1] - ns[b]):
            p, lo, hi = got[(b, k)]
            assert p == parts[k]
            keys.extend(range(lo, hi))
        assert keys == list(range(int(lens[b])))


def test_schedule_even_halves():
    """With the fixed cost split over both ends of a sequence, equal sequences
    over twice as many parts are cut exactly in half: every part holds one
    piece of half a sequence (hand-checked: 128 x 4096 keys, 32-key units,
    fixed cost 5, 256 parts: T = 128 x 266 / 256 = 133 half units)."""
    lens = np.full(128, 4096)
    meta, ns = oracle.schedule(lens, num_parts=256, fixed_cost=5, unit_tokens=32)
    np.testing.assert_array_equal(ns, np.arange(0, 257, 2))
    for p in range(256):
        b, half = divmod(p, 2)
        assert tuple(meta[p, :4]) == (b, 2048 * half, b, 2048 * (half + 1))


@pytest.mark.parametrize("B,num_parts", [(32, 256), (32, 128), (64, 128), (6, 48)])
@pytest.mark.parametrize("fixed_cost", [1, 2, 3, 4, 5])
def test_schedule_equal_sequences_whole_groups(B, num_parts, fixed_cost):
    """The line is shared evenly, so a batch of equal sequences whose count
    divides the part count splits into whole groups of num_parts / B parts
    per sequence, for any fixed cost: no part spans two sequences and none is
    left empty (hand-checked: 32 x 4096 keys, fixed cost 3, 256 parts: each
    sequence spans 262 half units = 8 parts of 32.75; its first piece ends at
    the first unit midpoint past 32.75, unit 15, so pieces hold 15, 16, 17,
    16, 16, 17, 16 and 15 units)."""
    lens = np.full(B, 4096)
    meta, ns = oracle.schedule(lens, num_parts=num_parts, fixed_cost=fixed_cost, unit_tokens=32)
    per = num_parts // B
    np.testing.assert_array_equal(ns, np.arange(0, num_parts + 1, per))
    for p in range(num_parts):
        b = p // per
        assert meta[p, 0] == b and meta[p, 2] == b, (p, meta[p])
    if (B, num_parts, fixed_cost) == (32, 256, 3):
        units = [(int(meta[p, 3]) - int(meta[p, 1])) // 32 for p in range(8)]
        assert units == [15, 16, 17, 16, 16, 17, 16, 15]


def test_schedule_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.schedule([1, 2], num_parts=0, fixed_cost=1)
    with pytest.raises(ValueError):
        oracle.schedule([1, 2], num_parts=4, fixed_cost=0)
    with pytest.raises(ValueError):
        oracle.schedule([1, -2], num_parts=4, fixed_cost=1)


# --------------------------------------------------------------------------
# fp16 inputs (the element type one page lists beside bf16)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_widening_matches_numpy_for_every_bit_pattern(dtype):
    """The oracle's widening of all 65536 patterns equals numpy's (fp16) or the
    bf16-is-the-top-half-of-binary32 rule evaluated by numpy (bf16)."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.widen(bits, dtype)
    ref = to64(bits, dtype)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("seed", range(12))
def test_fp16_oracle_matches_dense_brute_force(seed):
    w = random_tiny(seed, dtype="fp16")
    out, lse = run_oracle(w)
    rout, rlse = dense_reference(w)
    assert_close(lse, rlse, rtol=1e-11, atol=1e-11)
    assert_close(out, rout, rtol=1e-9, atol=1e-11)


def test_fp16_and_bf16_read_the_same_bits_differently():
    """The same bit patterns give different results per dtype (the dtype is
    really passed through), and fp16 inputs of bf16-representable values
    give the bf16 result."""
    w = random_tiny(3, dtype="fp16")
    o16, l16 = run_oracle(w)
    o_b, l_b = oracle.decode(w.q, w.kcache, w.block_table, w.seqlens, causal=w.causal,
                             scale=w.scale, dtype="bf16")
    assert not np.allclose(np.nan_to_num(l16), np.nan_to_num(l_b))
    # values exact in both formats: small integers / 4
    rng = np.random.default_rng(7)
    vals = rng.integers(-8, 9, size=w.kcache.shape).astype(np.float32) / 4
    qv = rng.integers(-8, 9, size=w.q.shape).astype(np.float32) / 4
    o1, l1 = oracle.decode(qv.astype(np.float16).view(np.uint16), vals.astype(np.float16).view(np.uint16),
                           w.block_table, w.seqlens, causal=w.causal, scale=w.scale, dtype="fp16")
    o2, l2 = oracle.decode(bf16_bits(qv), bf16_bits(vals), w.block_table, w.seqlens,
                           causal=w.causal, scale=w.scale, dtype="bf16")
    assert_close(o1, o2, rtol=0, atol=0)
    assert_close(l1, l2, rtol=0, atol=0)
