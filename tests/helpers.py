"""Test helpers: raw-code views of torch tensors and oracle-side pool building.

The oracle pools are built only with ``oracle.paged`` (its own address map and
append); nothing here touches the HIP library.
"""
from __future__ import annotations

import numpy as np

import oracle
from workloads import POISON, Workload


def codes(t, dtype: str) -> np.ndarray:
    """Raw element codes of a CPU/GPU torch tensor as a numpy array."""
    import torch
    t = t.detach()
    if t.is_cuda:
        t = t.cpu()
    if dtype == "f32":
        return t.contiguous().view(torch.int32).numpy().view(np.uint32)
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8":
        return t.contiguous().view(torch.uint8).numpy()
    raise ValueError(dtype)


def poisoned_pool(w: Workload) -> np.ndarray:
    shape = (w.num_blocks, w.block_size, w.n_kv_heads, w.head_dim)
    return np.full(shape, POISON[w.cache_dtype])


def oracle_slots(w: Workload, which: str) -> np.ndarray:
    if which == "res":
        return oracle.paged.slot_mapping(w.block_tables, w.res_start, w.res_len, w.block_size)
    return oracle.paged.slot_mapping(w.block_tables, w.new_start, w.new_len, w.block_size)


def oracle_pools(w: Workload, include_new: bool = True):
    """Pools after appending the resident tokens (and the new ones if asked)."""
    pk, pv = poisoned_pool(w), poisoned_pool(w)
    src = w.src_dtype
    steps = [("res", w.res_k, w.res_v)] + ([("new", w.new_k, w.new_v)] if include_new else [])
    for which, k, v in steps:
        slots = oracle_slots(w, which)
        oracle.paged.kv_append(pk, codes(k, src), slots, w.block_size, src, w.cache_dtype, w.k_scale)
        oracle.paged.kv_append(pv, codes(v, src), slots, w.block_size, src, w.cache_dtype, w.v_scale)
    return pk, pv


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
