"""Test helpers: raw-code views of torch tensors and oracle-side pool building.

The oracle pools are built only with ``oracle.paged`` (its own address map and
append); nothing here touches the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import POISON, Workload, codes  # noqa: F401  (codes re-exported)


def poisoned_pool(w: Workload) -> np.ndarray:
    shape = (w.num_blocks, w.block_size, w.n_kv_heads, w.head_dim)
    return np.full(shape, POISON[w.cache_dtype])


def oracle_slots(w: Workload, which: str) -> np.ndarray:
    if which == "res":
        return oracle.paged.slot_mapping(w.block_tables, w.res_start, w.res_len, w.block_size)
    return oracle.paged.slot_mapping(w.block_tables, w.new_start, w.new_len, w.block_size)


def oracle_pools(w: Workload, include_new: bool = True, seqs=None):
    """Pools after appending the resident tokens (and the new ones if asked).

    With ``seqs`` only those sequences' tokens are appended (plus the sequence
    that writes a shared prefix, when a listed sequence reads it).
    """
    pk, pv = poisoned_pool(w), poisoned_pool(w)
    src = w.src_dtype
    if seqs is None:
        seqs = list(range(w.num_seqs))
    seqs = sorted(set(int(s) for s in seqs))
    if w.shared_prefix_seqs and any(s in w.shared_prefix_seqs for s in seqs):
        seqs = sorted(set(seqs) | {w.shared_prefix_seqs[0]})
    steps = [("res", w.res_start, w.res_len, w.res_k, w.res_v)]
    if include_new:
        steps.append(("new", w.new_start, w.new_len, w.new_k, w.new_v))
    for _, start, lens, k, v in steps:
        cu = w.cu(lens)
        idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]) if seqs else np.zeros(0, int)
        if idx.size == 0:
            continue
        slots = oracle.paged.slot_mapping(w.block_tables[seqs], start[seqs], lens[seqs], w.block_size)
        ti = torch.as_tensor(idx, device=k.device)
        kc = codes(k.index_select(0, ti), src)
        vc = codes(v.index_select(0, ti), src)
        oracle.paged.kv_append(pk, kc, slots, w.block_size, src, w.cache_dtype, w.k_scale)
        oracle.paged.kv_append(pv, vc, slots, w.block_size, src, w.cache_dtype, w.v_scale)
    return pk, pv


def oracle_pools_int4(w: Workload, include_new: bool = True, seqs=None):
    """INT4 pools (packed K, packed V, value scales) after the appends, as
    ``oracle_pools`` does for the other dtypes."""
    from workloads import INT4_SCALE_POISON
    shape = (w.num_blocks, w.block_size, w.n_kv_heads, w.head_dim // 2)
    pk = np.full(shape, POISON["int4"], np.uint8)
    pv = np.full(shape, POISON["int4"], np.uint8)
    ps = np.full((w.num_blocks, w.n_kv_heads, w.block_size), INT4_SCALE_POISON,
                 np.uint32).view(np.float32)
    src = w.src_dtype
    if seqs is None:
        seqs = list(range(w.num_seqs))
    seqs = sorted(set(int(s) for s in seqs))
    if w.shared_prefix_seqs and any(s in w.shared_prefix_seqs for s in seqs):
        seqs = sorted(set(seqs) | {w.shared_prefix_seqs[0]})
    steps = [(w.res_start, w.res_len, w.res_k, w.res_v)]
    if include_new:
        steps.append((w.new_start, w.new_len, w.new_k, w.new_v))
    for start, lens, k, v in steps:
        cu = w.cu(lens)
        idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]) if seqs else np.zeros(0, int)
        if idx.size == 0:
            continue
        slots = oracle.paged.slot_mapping(w.block_tables[seqs], start[seqs], lens[seqs], w.block_size)
        ti = torch.as_tensor(idx, device=k.device)
        oracle.paged.kv_append_int4(pk, pv, ps, codes(k.index_select(0, ti), src),
                                    codes(v.index_select(0, ti), src), slots, w.block_size, src,
                                    w.k_channel_scales)
    return pk, pv, ps


def oracle_decode_int4(w: Workload, pk, pv, ps, rows=None):
    """Oracle decode output for the decode rows of an INT4 workload (float64)."""
    rows = list(w.decode_rows) if rows is None else list(rows)
    qc = codes(w.q, w.q_dtype)
    cu = w.cu(w.q_lens)
    qd = np.zeros((w.num_seqs,) + qc.shape[1:], dtype=qc.dtype)
    for s in rows:
        qd[s] = qc[cu[s]]
    return oracle.paged.decode_int4(qd, w.q_dtype, pk, pv, ps, w.k_channel_scales,
                                    w.block_tables, w.context_lens, w.block_size, w.group_size,
                                    w.scale, rows=rows)


def blocks_of(w: Workload, seqs) -> np.ndarray:
    """Physical block ids read by the listed sequences."""
    ids = []
    for s in seqs:
        n = -(-int(w.context_lens[s]) // w.block_size)
        ids.extend(w.block_tables[s, :n].tolist())
    return np.unique(np.array(ids, dtype=np.int64))


def oracle_decode(w: Workload, pk, pv, rows=None):
    """Oracle decode output for the decode rows of ``w`` (float64)."""
    rows = list(w.decode_rows) if rows is None else list(rows)
    qc = codes(w.q, w.q_dtype)
    # decode rows own query rows cu[s] .. cu[s]+1; gather them in row order
    cu = w.cu(w.q_lens)
    qd = np.zeros((w.num_seqs,) + qc.shape[1:], dtype=qc.dtype)
    for s in rows:
        qd[s] = qc[cu[s]]
    return oracle.paged.decode(qd, w.q_dtype, pk, pv, w.cache_dtype, w.block_tables,
                               w.context_lens, w.block_size, w.group_size, w.scale,
                               w.k_scale, w.v_scale, rows=rows)


def oracle_prefill(w: Workload, pk, pv, rows=None):
    P = w.num_prefill_seqs
    cu = w.cu(w.q_lens[:P])
    qc = codes(w.q, w.q_dtype)[: cu[-1]]
    return oracle.paged.prefill_chunk(qc, w.q_dtype, cu, pk, pv, w.cache_dtype,
                                      w.block_tables[:P], w.context_lens[:P], w.block_size,
                                      w.group_size, w.scale, w.causal, w.k_scale, w.v_scale,
                                      rows=rows)


def normwise_rel(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """max|got - ref| / max|ref| over the last axis (one value per output row)."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)
