"""Paged-KV attention, written out from its definition (test infrastructure only).

Sources (the pages of the paged-KV study):

* [Batching] "3.3 Batching and memory management" (llm-learning-path tutorial),
  section "PagedAttention: the block table": the pool is cut into blocks of
  S_blk tokens; entry j of a sequence's block table names the physical block
  holding tokens [j*S_blk, (j+1)*S_blk); token p lives in block
  table[floor(p / S_blk)] at offset p mod S_blk; worked example with block
  size 4.  Section "Chunked prefill": a chunk's queries attend to a cache that
  already holds the earlier chunks.
* [KV-cache] "KV Cache: the memory bottleneck of LLM inference" (excerpt on
  the "PagedAttention" tag page), section 1.1: the output at step t is
  softmax(q_t K_{1:t}^T / sqrt(d_k)) V_{1:t}, with k_t, v_t appended to the
  cache first.  The KV-cache-optimisation excerpt on the same page gives the
  softmax(QK^T / sqrt(d_k)) V definition and grouped-query KV sharing.
* [Engineering] "From PagedAttention to Chunked Prefill" (ybb.press), section
  2.2: the block-by-block (online) softmax recurrence for m_i, l_i and O_i.
  The O_i update is printed with an inverse on the rescale factor; with an
  unnormalised accumulator the factor is e^{m_{i-1}-m_i} itself and the
  division by l happens once at the end -- that is the reading implemented in
  ``online_softmax`` below.  Section 3.2: mixed batches with query_len = 1
  rows beside query_len = chunk rows.

Conventions (readings of what the pages leave open):

* ``context_lens`` include the token(s) appended in the current step.
* A slot is the flattened address block * S_blk + offset; a negative slot
  means "skip".  Table rows are padded with -1, never read past ceil(ctx/S_blk).
* GQA: query head h reads KV head h // group_size.
* Chunk causality is bottom-right aligned: query i of a chunk of length L in a
  sequence of total length T sits at position T - L + i and sees keys j <= it.
* A query row that may see no key outputs zeros.
"""
from __future__ import annotations

import numpy as np

from . import codecs


# ----------------------------------------------------------------------------
# address map and append  ([Batching], "PagedAttention: the block table")
# ----------------------------------------------------------------------------

def slot_of(table_row, p: int, block_size: int) -> int:
    """Slot of logical position ``p``: block table[p // S_blk], offset p % S_blk."""
    block = int(table_row[p // block_size])
    if block < 0:
        return -1
    return block * block_size + p % block_size


def slot_mapping(block_tables, start_pos, lens, block_size: int) -> np.ndarray:
    """Slots of the tokens of segment s at positions start_pos[s] + i, i < lens[s]."""
    out = []
    for s in range(len(lens)):
        row = block_tables[s]
        p = int(start_pos[s]) + np.arange(int(lens[s]), dtype=np.int64)
        block = row[p // block_size].astype(np.int64)
        slot = block * block_size + p % block_size
        slot[block < 0] = -1
        out.append(slot)
    if not out:
        return np.zeros(0, np.int64)
    return np.concatenate(out).astype(np.int64)


def encode_tokens(new_codes, src_dtype: str, cache_dtype: str, scale: float = 1.0):
    """What a cache slot stores for a token: a bit copy, or e4m3(x * (1/scale))."""
    if cache_dtype == src_dtype:
        return np.array(new_codes, copy=True)
    if cache_dtype in ("fp8", "int8"):
        if src_dtype == "bf16":
            x = codecs.bf16_decode(new_codes).astype(np.float32)
        elif src_dtype == "f32":
            x = np.asarray(new_codes, dtype=np.uint32).view(np.float32)
        else:
            raise ValueError(src_dtype)
        with np.errstate(over="ignore", invalid="ignore"):
            y = (x * codecs.f32_inverse(scale)).astype(np.float32)   # one float32 product
        return codecs.e4m3_encode(y) if cache_dtype == "fp8" else codecs.int8_encode(y)
    raise ValueError((src_dtype, cache_dtype))


def kv_append(pool, new_codes, slots, block_size: int, src_dtype: str, cache_dtype: str,
              scale: float = 1.0):
    """Scatter: pool[slot // S_blk, slot % S_blk] = encode(new[i]) for slot >= 0.

    ``pool`` is modified in place and returned; every other byte is untouched.
    """
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    enc = encode_tokens(np.asarray(new_codes)[keep], src_dtype, cache_dtype, scale)
    b = slots[keep] // block_size
    o = slots[keep] % block_size
    pool[b, o] = enc
    return pool


def _src_f32(new_codes, src_dtype: str) -> np.ndarray:
    if src_dtype == "bf16":
        return codecs.bf16_decode(new_codes).astype(np.float32)
    if src_dtype == "f32":
        return np.asarray(new_codes, dtype=np.uint32).view(np.float32)
    raise ValueError(src_dtype)


def encode_int4_tokens(k_codes, v_codes, src_dtype: str, k_channel_scales):
    """INT4 rows of new tokens ([Engineering] 5.4, KIVI grouping).

    k_codes, v_codes [n, n_kv, hd] source codes; k_channel_scales [n_kv, hd].
    Keys: code = int4(k * (1 / s[head, channel])), one float32 product with the
    float32 inverse of the channel's scale.  Values: per (token, head) scale
    sigma = amax / 7, code = int4(v * (1 / sigma)).  Returns the packed K and V
    rows [n, n_kv, hd / 2] and sigma [n, n_kv] (float32).
    """
    xk = _src_f32(k_codes, src_dtype)
    xv = _src_f32(v_codes, src_dtype)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        kinv = (np.float32(1.0) / np.asarray(k_channel_scales, np.float32)).astype(np.float32)
        yk = (xk * kinv[None]).astype(np.float32)
        sigma, vinv = codecs.int4_token_scale(xv)
        yv = (xv * vinv[..., None]).astype(np.float32)
    return (codecs.int4_pack(codecs.int4_encode(yk)), codecs.int4_pack(codecs.int4_encode(yv)),
            sigma)


def kv_append_int4(pool_k, pool_v, v_scale_pool, k_codes, v_codes, slots, block_size: int,
                   src_dtype: str, k_channel_scales):
    """INT4 append: packed K/V rows into pool[slot // S_blk, slot % S_blk] and the
    token's value scales into v_scale_pool[slot // S_blk, h, slot % S_blk] (float32
    [num_blocks, n_kv, S_blk]: the scales of one head's tokens of a block are
    adjacent), for every slot >= 0.  All three are modified in place."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    pk, pv, sig = encode_int4_tokens(np.asarray(k_codes)[keep], np.asarray(v_codes)[keep],
                                     src_dtype, k_channel_scales)
    b, o = slots[keep] // block_size, slots[keep] % block_size
    pool_k[b, o] = pk
    pool_v[b, o] = pv
    v_scale_pool[b, :, o] = sig
    return pool_k, pool_v, v_scale_pool


def int4_seq_kv(pool_k, pool_v, v_scale_pool, table_row, ctx: int, block_size: int,
                k_channel_scales):
    """Dequantised K, V [ctx, n_kv, hd] (float64) of one sequence of an INT4 cache."""
    K = codecs.int4_unpack(materialise(pool_k, table_row, ctx, block_size))
    V = codecs.int4_unpack(materialise(pool_v, table_row, ctx, block_size))
    sig = materialise(np.swapaxes(v_scale_pool, 1, 2), table_row, ctx, block_size).astype(np.float64)
    s = np.asarray(k_channel_scales, np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return K * s[None], V * sig[..., None]


def decode_int4(q_codes, q_dtype, pool_k, pool_v, v_scale_pool, k_channel_scales, block_tables,
                context_lens, block_size: int, group_size: int, scale: float, rows=None):
    """Single-token decode over an INT4 cache: as ``decode`` on the dequantised K/V."""
    rows = range(len(context_lens)) if rows is None else rows
    q = codecs.decode(q_codes, q_dtype)
    n_q, hd = q.shape[1], q.shape[2]
    out = np.zeros((len(rows), n_q, hd), dtype=np.float64)
    for i, s in enumerate(rows):
        K, V = int4_seq_kv(pool_k, pool_v, v_scale_pool, block_tables[s], int(context_lens[s]),
                           block_size, k_channel_scales)
        for h in range(n_q):
            g = h // group_size
            out[i, h] = attention_two_pass(q[s, h][None, :], K[:, g, :], V[:, g, :], scale)[0]
    return out


def prefill_chunk_int4(q_codes, q_dtype, cu_seqlens_q, pool_k, pool_v, v_scale_pool,
                       k_channel_scales, block_tables, context_lens, block_size: int,
                       group_size: int, scale: float, causal: bool = True, rows=None):
    """Chunk attention over an INT4 cache: as ``prefill_chunk`` on the dequantised K/V."""
    q = codecs.decode(q_codes, q_dtype)
    out = np.zeros(q.shape, dtype=np.float64)
    n_q = q.shape[1]
    seqs = range(len(cu_seqlens_q) - 1) if rows is None else rows
    for s in seqs:
        a, b = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        L, T = b - a, int(context_lens[s])
        if L == 0:
            continue
        K, V = int4_seq_kv(pool_k, pool_v, v_scale_pool, block_tables[s], T, block_size,
                           k_channel_scales)
        pos = T - L + np.arange(L)
        keys = np.arange(T)
        allowed = (keys[None, :] <= pos[:, None]) if causal else np.ones((L, T), bool)
        for h in range(n_q):
            g = h // group_size
            out[a:b, h] = attention_two_pass(q[a:b, h], K[:, g, :], V[:, g, :], scale, allowed)
    return out


def copy_blocks(dst_pool, src_pool, pairs):
    """Whole-block copies: dst_pool[d] = src_pool[s] for every pair (s, d).

    [Batching] "Sharing and copy-on-write": before a sequence writes into a
    block that other sequences still reference (refcount > 1), the block is
    copied to a fresh one and the writer's table entry is pointed at the copy;
    section "Scheduling policy and preemption": a preempted sequence's blocks
    are copied out to host memory and copied back (to any free blocks) when it
    resumes.  Both are this operation, within one pool or between a device
    pool and a host pool.  Pairs whose source or destination lies outside its
    pool are skipped; ``dst_pool`` is modified in place and returned, and no
    block that is not a destination changes.
    """
    for s_blk, d_blk in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= s_blk < src_pool.shape[0] and 0 <= d_blk < dst_pool.shape[0]:
            dst_pool[d_blk] = src_pool[s_blk].copy()
    return dst_pool


def materialise(pool, table_row, ctx: int, block_size: int):
    """Contiguous [ctx, n_kv, hd] codes of one sequence, gathered block by block."""
    n_blocks = -(-int(ctx) // block_size)
    if n_blocks == 0:
        return pool[:0, 0]
    parts = [pool[int(table_row[j])] for j in range(n_blocks)]
    return np.concatenate(parts, axis=0)[:ctx]


# ----------------------------------------------------------------------------
# attention by definition ([KV-cache] section 1.1): two passes over the scores
# ----------------------------------------------------------------------------

def attention_two_pass(q, K, V, scale: float, allowed=None):
    """softmax(scale * q K^T) V per query row, float64, two passes.

    q [R, d], K [n, d], V [n, d]; ``allowed`` [R, n] boolean (None = all).
    Pass 1 takes the row maximum over allowed keys, pass 2 exponentiates,
    sums and weights V, then divides by the sum.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    R, n = q.shape[0], K.shape[0]
    out = np.zeros((R, V.shape[1]), dtype=np.float64)
    if n == 0:
        return out
    s = np.float64(scale) * (q @ K.T)
    if allowed is None:
        allowed = np.ones((R, n), dtype=bool)
    for r in range(R):
        a = allowed[r]
        if not a.any():
            continue                                   # no key: zeros
        sr = s[r, a]
        m = sr.max()                                   # pass 1
        p = np.exp(sr - m)                             # pass 2
        out[r] = (p @ V[a]) / p.sum()
    return out


def _seq_kv(pool_k, pool_v, table_row, ctx, bs, cache_dtype, k_scale, v_scale):
    Kc = materialise(pool_k, table_row, ctx, bs)
    Vc = materialise(pool_v, table_row, ctx, bs)
    return (codecs.decode(Kc, cache_dtype, k_scale), codecs.decode(Vc, cache_dtype, v_scale))


def decode(q_codes, q_dtype, pool_k, pool_v, cache_dtype, block_tables, context_lens,
           block_size: int, group_size: int, scale: float, k_scale: float = 1.0,
           v_scale: float = 1.0, rows=None):
    """Single-token decode for every sequence (or the listed ``rows``).

    q_codes [B, n_q, hd] -> float64 [len(rows), n_q, hd].  Sequence s attends
    to its keys 0 .. context_lens[s]-1 (the appended token included).
    """
    rows = range(len(context_lens)) if rows is None else rows
    q = codecs.decode(q_codes, q_dtype)
    n_q, hd = q.shape[1], q.shape[2]
    out = np.zeros((len(rows), n_q, hd), dtype=np.float64)
    for i, s in enumerate(rows):
        ctx = int(context_lens[s])
        K, V = _seq_kv(pool_k, pool_v, block_tables[s], ctx, block_size, cache_dtype,
                       k_scale, v_scale)
        for h in range(n_q):
            g = h // group_size
            out[i, h] = attention_two_pass(q[s, h][None, :], K[:, g, :], V[:, g, :], scale)[0]
    return out


def prefill_chunk(q_codes, q_dtype, cu_seqlens_q, pool_k, pool_v, cache_dtype, block_tables,
                  context_lens, block_size: int, group_size: int, scale: float,
                  causal: bool = True, k_scale: float = 1.0, v_scale: float = 1.0, rows=None):
    """Chunk attention: the L_s queries of sequence s sit at T_s - L_s + i.

    q_codes [sum L, n_q, hd] -> float64, same shape (only ``rows`` filled when given).
    With ``causal`` query i sees keys j <= T_s - L_s + i, else all j < T_s.
    """
    q = codecs.decode(q_codes, q_dtype)
    out = np.zeros(q.shape, dtype=np.float64)
    n_q = q.shape[1]
    seqs = range(len(cu_seqlens_q) - 1) if rows is None else rows
    for s in seqs:
        a, b = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        L, T = b - a, int(context_lens[s])
        if L == 0:
            continue
        K, V = _seq_kv(pool_k, pool_v, block_tables[s], T, block_size, cache_dtype,
                       k_scale, v_scale)
        pos = T - L + np.arange(L)
        keys = np.arange(T)
        allowed = (keys[None, :] <= pos[:, None]) if causal else np.ones((L, T), bool)
        for h in range(n_q):
            g = h // group_size
            out[a:b, h] = attention_two_pass(q[a:b, h], K[:, g, :], V[:, g, :], scale, allowed)
    return out


# ----------------------------------------------------------------------------
# the recurrences the kernels use; pinned against the definition above
# ----------------------------------------------------------------------------

def online_softmax(q, K, V, scale: float, block_len: int):
    """[Engineering] section 2.2, block by block, unnormalised accumulator.

    For key block i with scores S_i:  m_i = max(m_{i-1}, rowmax S_i);
    l_i = e^{m_{i-1}-m_i} l_{i-1} + rowsum e^{S_i - m_i};
    O~_i = e^{m_{i-1}-m_i} O~_{i-1} + e^{S_i - m_i} V_i;  output O~_N / l_N.
    Returns (output, m_N, l_N, O~_N) for a single query row q [d].
    """
    q = np.asarray(q, np.float64)
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1], dtype=np.float64)
    for start in range(0, K.shape[0], block_len):
        Kb, Vb = K[start:start + block_len], V[start:start + block_len]
        s = scale * (Kb @ q)
        m_new = max(m, s.max())
        alpha = np.exp(m - m_new) if m != -np.inf else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ Vb
        m = m_new
    return acc / l, m, l, acc


def lse_merge(parts):
    """Merge split partials (m_k, l_k, O~_k) of one query row into the output.

    M = max_k m_k;  L = sum_k e^{m_k - M} l_k;  O = sum_k e^{m_k - M} O~_k / L.
    This is the combine step of the recurrence above applied to whole splits.
    """
    M = max(p[0] for p in parts)
    L = sum(np.exp(p[0] - M) * p[1] for p in parts)
    O = sum(np.exp(p[0] - M) * p[2] for p in parts)
    return O / L
