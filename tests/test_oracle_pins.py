"""Pins of the oracle against facts the pages and mathematics fix (CPU only).

Each test is chosen so that a plausible slip in the oracle -- a wrong index in
the address map, a transposed operand, a dropped rescale term, a mis-aligned
causal mask, a wrong GQA head map -- fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# P1: the worked block-table example (block size 4, A=[7,2,5], B=[3,4])
# --------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_probe_slot():
    g = _golden()
    bs = g["block_size"]
    pr = g["probe"]
    table = g["tables"][pr["seq"]]
    assert paged.slot_of(table, pr["pos"], bs) == pr["block"] * bs + pr["offset"]


def test_worked_example_pool_occupancy():
    """Append every token of A and B with a value naming (seq, pos); read the pool back."""
    g = _golden()
    bs, nb = g["block_size"], g["num_blocks"]
    names = sorted(g["tables"])
    tables = np.full((len(names), 3), -1, np.int32)
    for i, n in enumerate(names):
        tables[i, : len(g["tables"][n])] = g["tables"][n]
    lens = np.array([g["lengths"][n] for n in names], np.int32)
    poison = np.uint32(0xFFC0DEAD)
    pool = np.full((nb, bs, 1, 1), poison, dtype=np.uint32)
    slots = paged.slot_mapping(tables, np.zeros(2, np.int32), lens, bs)
    tag = np.concatenate([1000.0 * (i + 1) + np.arange(lens[i]) for i in range(2)])
    vals = tag.astype(np.float32).view(np.uint32).reshape(-1, 1, 1)
    paged.kv_append(pool, vals, slots, bs, "f32", "f32")
    got = pool.view(np.float32)[:, :, 0, 0]
    for blk, occ in g["occupancy"].items():
        blk = int(blk)
        s = names.index(occ["seq"])
        n = occ["last"] - occ["first"] + 1
        want = 1000.0 * (s + 1) + np.arange(occ["first"], occ["last"] + 1)
        np.testing.assert_array_equal(got[blk, :n], want)
        # the unused tail slots are never written
        assert (pool[blk, n:, 0, 0] == poison).all()
        assert bs - n == g["wasted_slots"].get(str(blk), 0)
    for blk in g["free_blocks"]:
        assert (pool[blk] == poison).all()


def test_worked_example_workload_matches_golden():
    from workloads import worked_example
    g = _golden()
    w = worked_example()
    assert w.block_size == g["block_size"] and w.num_blocks == g["num_blocks"]
    assert list(w.block_tables[0][:3]) == g["tables"]["A"]
    assert list(w.block_tables[1][:2]) == g["tables"]["B"]
    assert list(w.context_lens) == [g["lengths"]["A"], g["lengths"]["B"]]
    # the decode tokens are A.t9 and B.t5: slots 21 and 17
    np.testing.assert_array_equal(
        paged.slot_mapping(w.block_tables, w.new_start, w.new_len, w.block_size), [21, 17])


# --------------------------------------------------------------------------
# P2: brute force on tiny inputs (explicit loops over contiguous arrays)
# --------------------------------------------------------------------------

def _brute_attention(q, K, V, scale, n_allowed):
    """Attention of one query over keys 0..n_allowed-1 with math.exp loops."""
    if n_allowed == 0:
        return [0.0] * len(V[0])
    scores = [scale * sum(q[d] * K[j][d] for d in range(len(q))) for j in range(n_allowed)]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    tot = sum(w)
    return [sum(w[j] * V[j][d] for j in range(n_allowed)) / tot for d in range(len(V[0]))]


def _random_paged(rng, lens, bs, nkv, hd, spare=3):
    """Contiguous per-sequence K/V scattered into a randomly permuted pool."""
    need = [-(-L // bs) for L in lens]
    nb = sum(need) + spare
    perm = rng.permutation(nb)
    tables = np.full((len(lens), max(need + [1])), -1, np.int32)
    c = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[c:c + n]
        c += n
    Kc = [rng.standard_normal((L, nkv, hd)).astype(np.float32) for L in lens]
    Vc = [rng.standard_normal((L, nkv, hd)).astype(np.float32) for L in lens]
    pk = np.full((nb, bs, nkv, hd), np.uint32(0xFFC0DEAD))
    pv = pk.copy()
    slots = paged.slot_mapping(tables, np.zeros(len(lens), np.int32), np.array(lens), bs)
    if len(slots):
        paged.kv_append(pk, np.concatenate(Kc).view(np.uint32), slots, bs, "f32", "f32")
        paged.kv_append(pv, np.concatenate(Vc).view(np.uint32), slots, bs, "f32", "f32")
    return tables, pk, pv, Kc, Vc


@pytest.mark.parametrize("bs,group", [(3, 1), (4, 2), (5, 3)])
def test_decode_equals_brute_force(bs, group):
    rng = np.random.default_rng(7 + bs)
    lens = [1, bs, 2 * bs + 1, 11, 0]
    nkv, hd = 2, 5
    nq = nkv * group
    tables, pk, pv, Kc, Vc = _random_paged(rng, lens, bs, nkv, hd)
    # round trip: gathering back through the tables returns the contiguous data
    for s, L in enumerate(lens):
        np.testing.assert_array_equal(paged.materialise(pk, tables[s], L, bs).view(np.float32), Kc[s])
    q = rng.standard_normal((len(lens), nq, hd)).astype(np.float32)
    scale = 0.37
    out = paged.decode(q.view(np.uint32), "f32", pk, pv, "f32", tables, np.array(lens), bs,
                       group, scale)
    for s, L in enumerate(lens):
        for h in range(nq):
            g = h // group
            ref = _brute_attention(q[s, h].astype(float), Kc[s][:, g].astype(float),
                                   Vc[s][:, g].astype(float) if L else [[0.0] * hd], scale, L)
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-14)


def test_prefill_equals_brute_force_causal():
    rng = np.random.default_rng(11)
    bs, nkv, group, hd = 4, 2, 2, 6
    totals = [5, 9, 13]
    chunk = [5, 3, 6]           # first row has no prior context
    tables, pk, pv, Kc, Vc = _random_paged(rng, totals, bs, nkv, hd)
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = rng.standard_normal((cu[-1], nkv * group, hd)).astype(np.float32)
    out = paged.prefill_chunk(q.view(np.uint32), "f32", cu, pk, pv, "f32", tables,
                              np.array(totals), bs, group, 0.5, causal=True)
    for s, (T, L) in enumerate(zip(totals, chunk)):
        for i in range(L):
            pos = T - L + i
            for h in range(nkv * group):
                g = h // group
                ref = _brute_attention(q[cu[s] + i, h].astype(float), Kc[s][:, g].astype(float),
                                       Vc[s][:, g].astype(float), 0.5, pos + 1)
                np.testing.assert_allclose(out[cu[s] + i, h], ref, rtol=1e-12, atol=1e-14)
    # non-causal: every query sees the whole sequence
    outn = paged.prefill_chunk(q.view(np.uint32), "f32", cu, pk, pv, "f32", tables,
                               np.array(totals), bs, group, 0.5, causal=False)
    s, i, h = 1, 0, 3
    ref = _brute_attention(q[cu[s] + i, h].astype(float), Kc[s][:, h // group].astype(float),
                           Vc[s][:, h // group].astype(float), 0.5, totals[s])
    np.testing.assert_allclose(outn[cu[s] + i, h], ref, rtol=1e-12)


def test_chunking_does_not_change_prefill():
    """Chunked prefill: one chunk of 7 == chunks of 4 then 3 over the same cache."""
    rng = np.random.default_rng(5)
    bs, nkv, group, hd, T = 4, 1, 2, 4, 10
    tables, pk, pv, Kc, Vc = _random_paged(rng, [T], bs, nkv, hd)
    q = rng.standard_normal((7, 2, hd)).astype(np.float32)
    whole = paged.prefill_chunk(q.view(np.uint32), "f32", np.array([0, 7]), pk, pv, "f32",
                                tables, np.array([T]), bs, group, 0.3)
    first = paged.prefill_chunk(q[:4].view(np.uint32), "f32", np.array([0, 4]), pk, pv, "f32",
                                tables, np.array([T - 3]), bs, group, 0.3)
    second = paged.prefill_chunk(q[4:].view(np.uint32), "f32", np.array([0, 3]), pk, pv, "f32",
                                 tables, np.array([T]), bs, group, 0.3)
    np.testing.assert_array_equal(whole, np.concatenate([first, second]))


def test_decode_is_prefill_of_one():
    rng = np.random.default_rng(3)
    tables, pk, pv, _, _ = _random_paged(rng, [9, 4], 4, 2, 8)
    q = rng.standard_normal((2, 4, 8)).astype(np.float32)
    d = paged.decode(q.view(np.uint32), "f32", pk, pv, "f32", tables, np.array([9, 4]), 4, 2, 0.2)
    p = paged.prefill_chunk(q.view(np.uint32), "f32", np.array([0, 1, 2]), pk, pv, "f32",
                            tables, np.array([9, 4]), 4, 2, 0.2)
    np.testing.assert_array_equal(d, p)


# --------------------------------------------------------------------------
# P3: permutation invariance of the physical block ids
# --------------------------------------------------------------------------

def test_block_permutation_invariance():
    rng = np.random.default_rng(21)
    lens = [7, 16, 3, 30]
    bs, nkv, group, hd = 4, 2, 2, 8
    tables, pk, pv, _, _ = _random_paged(rng, lens, bs, nkv, hd)
    q = rng.standard_normal((len(lens), nkv * group, hd)).astype(np.float32).view(np.uint32)
    base = paged.decode(q, "f32", pk, pv, "f32", tables, np.array(lens), bs, group, 0.25)
    nb = pk.shape[0]
    pi = rng.permutation(nb)
    pk2, pv2 = np.empty_like(pk), np.empty_like(pv)
    pk2[pi] = pk
    pv2[pi] = pv
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    again = paged.decode(q, "f32", pk2, pv2, "f32", t2, np.array(lens), bs, group, 0.25)
    np.testing.assert_array_equal(base, again)
    # a wrong table (ids not permuted) must change the answer
    wrong = paged.decode(q, "f32", pk2, pv2, "f32", tables, np.array(lens), bs, group, 0.25)
    assert not np.array_equal(base, wrong)


# --------------------------------------------------------------------------
# P4: online (block-by-block) recurrence and split merge == two-pass definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("block_len", [1, 3, 16, 100])
def test_online_softmax_equals_two_pass(block_len):
    rng = np.random.default_rng(block_len)
    n, d = 97, 16
    q = rng.standard_normal(d) * 3
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    ref = paged.attention_two_pass(q[None], K, V, 0.7)[0]
    got, m, l, acc = paged.online_softmax(q, K, V, 0.7, block_len)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
    s = 0.7 * (K @ q)
    assert m == s.max()
    np.testing.assert_allclose(l, np.exp(s - s.max()).sum(), rtol=1e-13)


def test_inverse_rescale_reading_is_wrong():
    """The O update printed with an inverse factor does not reproduce attention."""
    rng = np.random.default_rng(0)
    q, K, V = rng.standard_normal(8), rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    ref = paged.attention_two_pass(q[None], K, V, 1.0)[0]
    m, l, acc = -np.inf, 0.0, np.zeros(8)
    for st in range(0, 40, 8):
        s = K[st:st + 8] @ q
        mn = max(m, s.max())
        a = np.exp(m - mn) if m != -np.inf else 0.0
        l = a * l + np.exp(s - mn).sum()
        acc = (1.0 / a if a else 0.0) * acc + np.exp(s - mn) @ V[st:st + 8]
        m = mn
    assert not np.allclose(acc / l, ref, rtol=1e-6)


def test_lse_merge_of_any_partition_equals_two_pass():
    rng = np.random.default_rng(4)
    n, d = 200, 12
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    ref = paged.attention_two_pass(q[None], K, V, 0.9)[0]
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, n), size=trial + 1, replace=False))
        bounds = [0] + cuts.tolist() + [n]
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            _, m, l, acc = paged.online_softmax(q, K[a:b], V[a:b], 0.9, 7)
            parts.append((m, l, acc))
        np.testing.assert_allclose(paged.lse_merge(parts), ref, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# P5: closed forms and the textbook special cases
# --------------------------------------------------------------------------

def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    tables, pk, pv, Kc, Vc = _random_paged(rng, [1, 1], 4, 2, 8)
    q = rng.standard_normal((2, 2, 8)).astype(np.float32).view(np.uint32)
    out = paged.decode(q, "f32", pk, pv, "f32", tables, np.array([1, 1]), 4, 1, 1.0)
    for s in range(2):
        np.testing.assert_array_equal(out[s], Vc[s][0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    tables, pk, pv, Kc, Vc = _random_paged(rng, [13], 4, 1, 8)
    q = np.zeros((1, 1, 8), np.float32).view(np.uint32)
    out = paged.decode(q, "f32", pk, pv, "f32", tables, np.array([13]), 4, 1, 1.0)
    np.testing.assert_allclose(out[0, 0], Vc[0][:, 0].astype(np.float64).mean(axis=0),
                               rtol=1e-14, atol=1e-16)


def test_one_hot_key_selects_its_value_exactly():
    """A key whose score beats the rest by > 800 takes all weight (e^-800 == 0)."""
    rng = np.random.default_rng(9)
    L, bs, nkv, group, hd = 23, 4, 2, 2, 8
    tables, pk, pv, Kc, Vc = _random_paged(rng, [L], bs, nkv, hd)
    target = 17
    direction = np.zeros(hd, np.float32)
    direction[3] = 1.0
    Kf = pk.view(np.float32)
    for j in range(L):
        b, o = tables[0][j // bs], j % bs
        Kf[b, o] = 0.0
    b, o = tables[0][target // bs], target % bs
    Kf[b, o, :, :] = 40.0 * direction
    q = np.tile(40.0 * direction, (1, nkv * group, 1)).astype(np.float32)
    out = paged.decode(q.view(np.uint32), "f32", pk, pv, "f32", tables, np.array([L]), bs,
                       group, 1.0)
    for h in range(nkv * group):
        np.testing.assert_array_equal(out[0, h], Vc[0][target, h // group].astype(np.float64))


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(12)
    lens, bs, nkv, group, hd = [9, 14], 4, 2, 3, 6
    tables, pk, pv, _, _ = _random_paged(rng, lens, bs, nkv, hd)
    q = rng.standard_normal((2, nkv * group, hd)).astype(np.float32).view(np.uint32)
    gqa = paged.decode(q, "f32", pk, pv, "f32", tables, np.array(lens), bs, group, 0.4)
    pk_r = np.repeat(pk, group, axis=2)
    pv_r = np.repeat(pv, group, axis=2)
    mha = paged.decode(q, "f32", pk_r, pv_r, "f32", tables, np.array(lens), bs, 1, 0.4)
    np.testing.assert_array_equal(gqa, mha)
    # and the head map matters: pairing q-head h with kv-head h % nkv differs
    pk_w = np.tile(pk, (1, 1, group, 1))
    pv_w = np.tile(pv, (1, 1, group, 1))
    wrong = paged.decode(q, "f32", pk_w, pv_w, "f32", tables, np.array(lens), bs, 1, 0.4)
    assert not np.array_equal(gqa, wrong)


def test_empty_context_gives_zeros():
    pk = np.full((2, 4, 1, 4), np.uint32(0xFFC0DEAD))
    out = paged.decode(np.ones((1, 1, 4), np.float32).view(np.uint32), "f32", pk, pk, "f32",
                       np.array([[-1]], np.int32), np.array([0]), 4, 1, 1.0)
    np.testing.assert_array_equal(out, 0.0)


def test_negative_slot_is_skipped_and_untouched_bytes_stay():
    pool = np.full((3, 2, 1, 2), np.uint16(0xFFC1))
    new = np.array([[[1, 2]], [[3, 4]], [[5, 6]]], np.uint16)
    paged.kv_append(pool, new, np.array([3, -1, 0]), 2, "bf16", "bf16")
    assert (pool[1, 1, 0] == [1, 2]).all() and (pool[0, 0, 0] == [5, 6]).all()
    untouched = np.ones(pool.shape[:2], bool)
    untouched[1, 1] = untouched[0, 0] = False
    assert (pool[untouched] == 0xFFC1).all()
