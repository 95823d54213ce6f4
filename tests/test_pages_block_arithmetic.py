"""The block arithmetic the pages print, checked against the workloads' block
bookkeeping and the oracle's address map, append and block copy.

Values come from tests/golden/batching_numbers.json ("3.3 Batching and memory
management": sections "Self-test", "Worked numbers" and "Code").  CPU only.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import workloads
from oracle import paged

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "batching_numbers.json")))


def test_self_test_blocks_and_waste():
    """A 1,000-token sequence in blocks of 16: 63 blocks, 1,008 slots, 8 wasted."""
    g = GOLDEN["self_test"]
    n, bs = g["tokens"], g["block_size"]
    assert workloads._blocks_needed(n, bs) == g["blocks"]
    # the oracle's address map over the sequence's positions, with a table of
    # 63 distinct (permuted) blocks: every slot lands in a distinct cell, the
    # last block holds 1000 - 62 * 16 = 8 tokens, 8 slots stay unused
    table = np.random.default_rng(0).permutation(200)[: g["blocks"]]
    slots = paged.slot_mapping(table[None, :], np.array([0]), np.array([n]), bs)
    assert len(set(slots.tolist())) == n
    used = {}
    for s in slots:
        used.setdefault(int(s) // bs, set()).add(int(s) % bs)
    assert len(used) == g["blocks"] and set(used) == set(table.tolist())
    assert g["blocks"] * bs == g["slots"]
    assert g["slots"] - sum(len(v) for v in used.values()) == g["wasted_slots"]
    assert len(used[int(table[-1])]) == bs - g["wasted_slots"]


def test_worked_numbers():
    """Capacity of the pool and concurrent requests, contiguous against paged."""
    g = GOLDEN["worked_numbers"]
    # Llama-3-8B: 32 layers, 8 KV heads, 128 dims, K and V, 2 bytes each
    assert 2 * 32 * 8 * 128 * 2 == g["kv_bytes_per_token"]
    assert g["block_size"] * g["kv_bytes_per_token"] == g["block_bytes"]
    assert g["pool_bytes"] // g["block_bytes"] == g["pool_blocks"]
    assert g["pool_blocks"] * g["block_size"] == g["pool_tokens"]
    assert g["pool_tokens"] // g["contiguous_slots_per_request"] == g["contiguous_requests"]
    assert workloads._blocks_needed(g["paged_tokens_at_end"], g["block_size"]) == g["paged_blocks_at_end"]
    assert g["paged_blocks_at_end"] * g["block_size"] == g["paged_slots_at_end"]
    assert g["pool_tokens"] // g["paged_slots_at_end"] == g["paged_requests"]
    assert workloads._blocks_needed(g["shared_prompt_tokens"], g["block_size"]) == g["shared_prompt_blocks"]


def test_llama3_workload_follows_the_worked_numbers():
    """The Llama-3-8B-shaped decode workload: 800 shared prompt tokens are 50 blocks,
    stored once, and every sequence holds exactly ceil(ctx / 16) blocks."""
    g = GOLDEN["worked_numbers"]
    w = workloads.full(3)
    assert w.block_size == g["block_size"]
    assert w.shared_prefix_blocks == g["shared_prompt_blocks"]
    first = w.block_tables[w.shared_prefix_seqs[0], : g["shared_prompt_blocks"]]
    for s in w.shared_prefix_seqs:
        assert np.array_equal(w.block_tables[s, : g["shared_prompt_blocks"]], first)
    owned = []
    for s in range(w.num_seqs):
        n = math.ceil(int(w.context_lens[s]) / w.block_size)
        row = w.block_tables[s]
        assert (row[:n] >= 0).all() and (row[n:] < 0).all()
        owned.extend(row[:n].tolist())
    # shared blocks are the only ids held by more than one sequence
    ids, counts = np.unique(owned, return_counts=True)
    assert set(ids[counts > 1].tolist()) == set(first.tolist())
    assert (counts[counts > 1] == len(w.shared_prefix_seqs)).all()


class _Allocator:
    """The page's allocator rules, restated: a free list taken from its end,
    a reference count per block; fork shares every block; appending into a full
    last block takes a new one; appending into a shared last block first copies
    it to a new block (copy-on-write).  Returns the (src, dst) block copies the
    data side must perform."""

    def __init__(self, num_blocks, bs):
        self.bs, self.free, self.ref = bs, list(range(num_blocks)), [0] * num_blocks
        self.tables, self.lens = {}, {}

    def _take(self):
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def add(self, sid, n):
        self.tables[sid] = [self._take() for _ in range(-(-n // self.bs))]
        self.lens[sid] = n

    def fork(self, parent, child):
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, sid):
        t, n, copies = self.tables[sid], self.lens[sid], []
        if n % self.bs == 0:
            t.append(self._take())
        elif self.ref[t[-1]] > 1:
            self.ref[t[-1]] -= 1
            new = self._take()
            copies.append((t[-1], new))
            t[-1] = new
        self.lens[sid] = n + 1
        return copies

    def release(self, sid):
        for b in self.tables.pop(sid):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[sid]


def test_allocator_demo_fork_and_append():
    """Replay of the page's allocator demo on the oracle's data path: a 6-token prompt
    in blocks of 4 (2 blocks, the last half full), two forked samples, each appending
    its 7th token.  Each sample's write is preceded by a copy of the shared last prompt
    block (oracle.paged.copy_blocks) and lands in that copy (oracle.paged.kv_append
    through its own slot map); the parent and the other sample read their tokens
    unchanged, and the first block stays shared."""
    g = GOLDEN["allocator_demo"]
    bs, nb = g["block_size"], g["num_blocks"]
    al = _Allocator(nb, bs)
    al.add("p", g["prompt_tokens"])
    assert len(al.tables["p"]) == g["prompt_blocks"]
    al.fork("p", "s1")
    al.fork("p", "s2")
    rng = np.random.default_rng(5)
    nkv, hd = 2, 8
    pool = np.full((nb, bs, nkv, hd), 0xFFC1, np.uint16)           # bf16 NaN poison
    prompt = rng.integers(0, 0x7F00, size=(g["prompt_tokens"], nkv, hd)).astype(np.uint16)
    table_p = np.array([al.tables["p"]])
    paged.kv_append(pool, prompt, paged.slot_mapping(table_p, np.array([0]),
                                                     np.array([g["prompt_tokens"]]), bs),
                    bs, "bf16", "bf16")
    new_tok = {}
    for s in ("s1", "s2"):
        copies = al.append(s)
        assert len(copies) == 1 and copies[0][0] == al.tables["p"][-1]   # the half-full block
        paged.copy_blocks(pool, pool, copies)
        new_tok[s] = rng.integers(0, 0x7F00, size=(1, nkv, hd)).astype(np.uint16)
        slot = paged.slot_mapping(np.array([al.tables[s]]), np.array([g["prompt_tokens"]]),
                                  np.array([1]), bs)
        paged.kv_append(pool, new_tok[s], slot, bs, "bf16", "bf16")
    # each sample has a private last block, the first block is shared by all three
    lasts = {al.tables[s][-1] for s in ("p", "s1", "s2")}
    assert len(lasts) == 3
    assert al.tables["s1"][0] == al.tables["s2"][0] == al.tables["p"][0]
    # the data: the parent still reads its 6 tokens, each sample the prompt + its token
    np.testing.assert_array_equal(paged.materialise(pool, al.tables["p"], 6, bs), prompt)
    for s in ("s1", "s2"):
        seq = paged.materialise(pool, al.tables[s], 7, bs)
        np.testing.assert_array_equal(seq[:6], prompt)
        np.testing.assert_array_equal(seq[6], new_tok[s][0])
    # the half-full block of the parent still has its two free slots poisoned
    assert (pool[al.tables["p"][-1], 2:] == 0xFFC1).all()
    al.release("p")
    assert al.ref[al.tables["s1"][0]] == 2           # the first block: shared by the samples
    assert al.ref[al.tables["s1"][-1]] == al.ref[al.tables["s2"][-1]] == 1
    assert len(al.free) == nb - 3                    # first block + two private copies
