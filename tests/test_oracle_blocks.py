"""Pins of the oracle's block copy (copy-on-write and swap), from the scenarios the pages
describe ("3.3 Batching and memory management", sections "Sharing and copy-on-write" and
"Scheduling policy and preemption"), checked through the independent address map and
attention definitions.
"""
from __future__ import annotations

import numpy as np

from oracle import paged

BS, NKV, HD = 4, 2, 8


def _pool(nb, rng):
    return rng.integers(0, 1 << 16, size=(nb, BS, NKV, HD)).astype(np.uint16)


def test_copy_on_write_for_parallel_sampling():
    """n samples share a 6-token prompt (blocks [3, 7], the last one half full); sample 1
    writes its 7th token: the shared half block is copied to free block 5 first."""
    rng = np.random.default_rng(1)
    pool = _pool(8, rng)
    tables = np.array([[3, 7], [3, 7], [3, 7]])
    before = [paged.materialise(pool, tables[i], 6, BS) for i in range(3)]
    untouched = {b: pool[b].copy() for b in range(8) if b != 5}
    paged.copy_blocks(pool, pool, [(7, 5)])
    tables[1, 1] = 5
    new = rng.integers(0, 1 << 16, size=(1, NKV, HD)).astype(np.uint16)
    slot = paged.slot_of(tables[1], 6, BS)
    assert slot == 5 * BS + 2
    paged.kv_append(pool, new, [slot], BS, "bf16", "bf16")
    for i in (0, 2):   # the other samples see exactly the prompt, still in block 7
        assert np.array_equal(paged.materialise(pool, tables[i], 6, BS), before[i])
    seq1 = paged.materialise(pool, tables[1], 7, BS)
    assert np.array_equal(seq1[:6], before[1]) and np.array_equal(seq1[6], new[0])
    for b, v in untouched.items():
        assert np.array_equal(pool[b], v)


def test_swap_out_and_back_in_to_other_blocks():
    """Preemption by swapping: the sequence's blocks go to a host pool, the device blocks
    are reused by others, and the sequence resumes in different device blocks with the
    same attention output, bit for bit."""
    rng = np.random.default_rng(2)
    dev = np.zeros((10, BS, NKV, HD))
    table = np.array([[6, 1, 8]])
    ctx = np.array([11])
    q = rng.standard_normal((1, NKV, HD)).astype(np.float32).view(np.uint32)
    pk = rng.standard_normal(dev.shape).astype(np.float32).view(np.uint32)
    pv = rng.standard_normal(dev.shape).astype(np.float32).view(np.uint32)
    out0 = paged.decode(q, "f32", pk, pv, "f32", table, ctx, BS, 1, 0.3)
    host_k = np.zeros((3,) + pk.shape[1:], pk.dtype)
    host_v = np.zeros_like(host_k)
    paged.copy_blocks(host_k, pk, [(6, 0), (1, 1), (8, 2)])
    paged.copy_blocks(host_v, pv, [(6, 0), (1, 1), (8, 2)])
    pk[[6, 1, 8]] = 0xFFC0DEAD               # reused by other sequences meanwhile
    pv[[6, 1, 8]] = 0xFFC0DEAD
    paged.copy_blocks(pk, host_k, [(0, 2), (1, 9), (2, 4)])
    paged.copy_blocks(pv, host_v, [(0, 2), (1, 9), (2, 4)])
    out1 = paged.decode(q, "f32", pk, pv, "f32", np.array([[2, 9, 4]]), ctx, BS, 1, 0.3)
    assert np.array_equal(out0, out1)


def test_out_of_range_pairs_are_skipped():
    rng = np.random.default_rng(3)
    pool = _pool(4, rng)
    ref = pool.copy()
    paged.copy_blocks(pool, pool, [(-1, 2), (0, 4), (9, 1), (1, -3)])
    assert np.array_equal(pool, ref)
    paged.copy_blocks(pool, pool, [(0, 3), (2, 1)])
    assert np.array_equal(pool[3], ref[0]) and np.array_equal(pool[1], ref[2])
    assert np.array_equal(pool[0], ref[0]) and np.array_equal(pool[2], ref[2])
