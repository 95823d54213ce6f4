"""Seeded synthetic workloads for the paged-KV hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds only *draws* and *allocation bookkeeping*: sequence lengths, which
physical block ids each sequence owns (a random permutation of the pool, with
an optional shared prefix), and the random K/V/Q values.  It computes no slot
addresses and no attention: each side (the oracle and the HIP library) derives
those from the block tables with its own code.

Workload shapes follow the synthetic configurations of the paged-attention
study: a tiny fp32 case that reproduces the block-size-4 worked example of the
"Batching and memory management" tutorial (ch. 3.3, section "PagedAttention:
the block table"), Llama-2-7B-shaped MHA decode, Llama-3-8B-shaped GQA decode
with a shared 800-token (50-block) prompt prefix, a long-tail ragged decode
with 128K-token sequences (bf16 and fp8-e4m3 KV), and a chunked-prefill mixed
step.  The pages measure on no dataset; these draws stand in for real traffic.

Conventions
-----------
* ``context_lens[s]`` counts every token of sequence ``s`` *including* the
  token(s) appended in the current step.
* Tokens are described as one segment per sequence: ``(start_pos[s], len[s])``
  with the values stored flat in segment order, ``[sum(len), n_kv, head_dim]``.
* Raw element codes are stored: float32 values for "f32", uint16 bit patterns
  for "bf16" (rounded from float32 draws by round-to-nearest-even, via torch).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

def codes(t, dtype: str) -> np.ndarray:
    """Raw element codes of a CPU or GPU torch tensor as a numpy array (a bit view,
    copied to the host when the tensor lives on the GPU)."""
    import torch
    t = t.detach()
    if t.is_cuda:
        t = t.cpu()
    if dtype == "f32":
        return t.contiguous().view(torch.int32).numpy().view(np.uint32)
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if dtype in ("fp8", "int8"):
        return t.contiguous().view(torch.uint8).numpy()
    raise ValueError(dtype)


# Bit patterns used to fill the pool before anything is appended.  They are
# NaNs, so any read of a slot that no token owns shows up in the results.
POISON = {"f32": np.uint32(0xFFC0DEAD), "bf16": np.uint16(0xFFC1), "fp8": np.uint8(0x7F),
          "int8": np.uint8(0x80),       # int8: -128, outside the code range [-127, 127]
          # int4: every byte is a valid code pair, so the poison that shows is the
          # NaN in the value-scale pool at every slot no token owns
          "int4": np.uint8(0x77)}
INT4_SCALE_POISON = np.uint32(0xFFC0DEAD)
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1, "int4": 0.5}


@dataclasses.dataclass
class Workload:
    name: str
    cache_dtype: str            # "f32" | "bf16" | "fp8" | "int8" | "int4"
    q_dtype: str                # "f32" | "bf16"   (output dtype == q dtype)
    src_dtype: str              # dtype of K/V handed to the append call
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray    # int32 [B]
    block_tables: np.ndarray    # int32 [B, max_blocks], -1 padded
    q_lens: np.ndarray          # int32 [B]  (1 for decode rows)
    # tokens written before the step (start, len per sequence) and in the step
    res_start: np.ndarray
    res_len: np.ndarray
    new_start: np.ndarray
    new_len: np.ndarray
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    k_channel_scales: object = None   # int4: float32 [n_kv, hd], one key scale per channel
    causal: bool = True
    num_prefill_seqs: int = 0   # rows [0, num_prefill_seqs) are prefill chunks
    shared_prefix_seqs: tuple = ()
    shared_prefix_blocks: int = 0
    seed: int = 0
    value_std: float = 0.5
    # values (torch tensors; CPU or device) -- filled by draw_values()
    q: object = None            # [sum(q_lens), n_q, hd]
    res_k: object = None        # [sum(res_len), n_kv, hd]
    res_v: object = None
    new_k: object = None        # [sum(new_len), n_kv, hd]
    new_v: object = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def cu(self, lens: np.ndarray) -> np.ndarray:
        out = np.zeros(lens.shape[0] + 1, dtype=np.int32)
        np.cumsum(lens, out=out[1:])
        return out

    @property
    def decode_rows(self) -> range:
        return range(self.num_prefill_seqs, self.num_seqs)


# --------------------------------------------------------------------------
# structure draws
# --------------------------------------------------------------------------

def _blocks_needed(n_tokens: int, bs: int) -> int:
    # a sequence holds ceil(n/bs) blocks: a new block is taken only when the
    # last one is full (allocation bookkeeping, not an address computation)
    return -(-int(n_tokens) // bs)


def _assign_blocks(rng, ctx, bs, shared_idx=(), shared_blocks=0, spare=0):
    """Give every sequence ceil(ctx/bs) physical ids from a random permutation.

    Sequences listed in ``shared_idx`` take the same first ``shared_blocks``
    ids (refcount = len(shared_idx)); ``spare`` extra ids stay free.
    """
    B = len(ctx)
    need = [_blocks_needed(c, bs) for c in ctx]
    shared_set = set(int(i) for i in shared_idx)
    own = [n - (shared_blocks if s in shared_set else 0) for s, n in enumerate(need)]
    total = sum(own) + (shared_blocks if shared_set else 0) + spare
    perm = rng.permutation(total).astype(np.int32)
    maxb = max(need) if need else 1
    tables = np.full((B, max(maxb, 1)), -1, dtype=np.int32)
    cursor = 0
    shared_ids = perm[cursor:cursor + shared_blocks] if shared_set else perm[:0]
    cursor += len(shared_ids)
    for s in range(B):
        row = []
        if s in shared_set:
            row.extend(shared_ids.tolist())
        row.extend(perm[cursor:cursor + own[s]].tolist())
        cursor += own[s]
        tables[s, :len(row)] = row
    return tables, total


def _decode_segments(ctx):
    """Resident tokens [0, ctx-1), one new token at ctx-1 (zero-length rows stay empty)."""
    ctx = np.asarray(ctx, dtype=np.int32)
    new_len = (ctx > 0).astype(np.int32)
    return (np.zeros_like(ctx), ctx - new_len, ctx - new_len, new_len)


# --------------------------------------------------------------------------
# value draws
# --------------------------------------------------------------------------

def _gen(device: str, seed: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _draw(g, shape, dtype: str, std: float, device: str):
    import torch
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return x.to(torch.bfloat16)      # round-to-nearest-even
    raise ValueError(dtype)


def draw_values(w: Workload, device: str = "cpu") -> Workload:
    """Fill q / res_k / res_v / new_k / new_v (draw order: q, K, V, new K, new V)."""
    g = _gen(device, w.seed)
    nq, nkv, hd = w.n_q_heads, w.n_kv_heads, w.head_dim
    w.q = _draw(g, (int(w.q_lens.sum()), nq, hd), w.q_dtype, w.value_std, device)
    w.res_k = _draw(g, (int(w.res_len.sum()), nkv, hd), w.src_dtype, w.value_std, device)
    w.res_v = _draw(g, (int(w.res_len.sum()), nkv, hd), w.src_dtype, w.value_std, device)
    w.new_k = _draw(g, (int(w.new_len.sum()), nkv, hd), w.src_dtype, w.value_std, device)
    w.new_v = _draw(g, (int(w.new_len.sum()), nkv, hd), w.src_dtype, w.value_std, device)
    if w.cache_dtype in ("fp8", "int8"):
        # per-tensor scales: amax / 448 (largest finite e4m3 magnitude) or amax / 127, fp32
        import torch
        top = np.float32(448.0 if w.cache_dtype == "fp8" else 127.0)
        def amax(*ts):   # over the rows there are (a batch of empty contexts has none: scale 1)
            m = [t.float().abs().amax() for t in ts if t.numel()]
            return float(torch.stack(m).max()) if m else float(top)
        w.k_scale = float(np.float32(amax(w.res_k, w.new_k)) / top)
        w.v_scale = float(np.float32(amax(w.res_v, w.new_v)) / top)
    if w.cache_dtype == "int4":
        # per-channel key scales (the caller's calibration): amax over every key
        # of the workload per (KV head, channel) / 7, fp32
        import torch
        ka = w.res_k.float().abs().amax(dim=0)
        if w.new_k.numel():
            ka = torch.maximum(ka, w.new_k.float().abs().amax(dim=0))
        w.k_channel_scales = (ka.cpu().numpy().astype(np.float32) / np.float32(7.0)).astype(np.float32)
    return w


# --------------------------------------------------------------------------
# the five configurations (and reduced-size variants for full oracle checks)
# --------------------------------------------------------------------------

def worked_example() -> Workload:
    """Block size 4, A = 10 tokens in blocks [7, 2, 5], B = 6 tokens in [3, 4].

    Blocks 0, 1, 6 stay free.  Each sequence decodes one token, so A's t9 and
    B's t5 are the appended tokens and every other token is resident.
    """
    ctx = np.array([10, 6], dtype=np.int32)
    tables = np.array([[7, 2, 5], [3, 4, -1]], dtype=np.int32)
    rs, rl, ns, nl = _decode_segments(ctx)
    w = Workload(name="tiny-fp32", cache_dtype="f32", q_dtype="f32", src_dtype="f32",
                 n_q_heads=2, n_kv_heads=2, head_dim=64, block_size=4, num_blocks=8,
                 context_lens=ctx, block_tables=tables, q_lens=np.ones(2, np.int32),
                 res_start=rs, res_len=rl, new_start=ns, new_len=nl,
                 scale=1.0 / 8.0, seed=0, value_std=1.0)
    return w


def _decode_workload(name, rng, ctx, nq, nkv, hd, bs, cache_dtype, q_dtype, src_dtype,
                     shared_idx=(), shared_blocks=0, spare=0, seed=0):
    tables, nb = _assign_blocks(rng, ctx, bs, shared_idx, shared_blocks, spare)
    rs, rl, ns, nl = _decode_segments(ctx)
    shared_set = sorted(int(i) for i in shared_idx)
    # every sharer but the first finds the prefix already written
    for s in shared_set[1:]:
        rs[s] = shared_blocks * bs
        rl[s] = ctx[s] - 1 - rs[s]
    return Workload(name=name, cache_dtype=cache_dtype, q_dtype=q_dtype, src_dtype=src_dtype,
                    n_q_heads=nq, n_kv_heads=nkv, head_dim=hd, block_size=bs, num_blocks=nb,
                    context_lens=np.asarray(ctx, np.int32), block_tables=tables,
                    q_lens=np.ones(len(ctx), np.int32),
                    res_start=rs, res_len=rl, new_start=ns, new_len=nl,
                    scale=1.0 / math.sqrt(hd), shared_prefix_seqs=tuple(shared_set),
                    shared_prefix_blocks=shared_blocks if shared_set else 0, seed=seed)


def llama2_7b_decode(batch=64, lo=128, hi=4096, seed=0) -> Workload:
    """MHA decode: 32 q / 32 kv heads, head_dim 128, block 16, bf16, ctx ~ U{lo..hi}."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    return _decode_workload("llama2-7b-decode", rng, ctx, 32, 32, 128, 16,
                            "bf16", "bf16", "bf16", seed=seed)


def llama3_8b_gqa_decode(batch=64, lo=2048, hi=8192, n_shared=19, prefix_tokens=800,
                         seed=0) -> Workload:
    """GQA-4 decode with a shared prompt prefix held once in the pool.

    ``n_shared`` sequences (a seeded choice) point their first
    ``prefix_tokens / 16`` table entries at the same physical blocks.
    """
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    bs = 16
    assert prefix_tokens % bs == 0 and prefix_tokens < lo
    shared = rng.choice(batch, size=n_shared, replace=False) if n_shared else ()
    return _decode_workload("llama3-8b-gqa-decode", rng, ctx, 32, 8, 128, bs,
                            "bf16", "bf16", "bf16", shared_idx=shared,
                            shared_blocks=prefix_tokens // bs, seed=seed)


def long_tail_decode(batch=256, median=1024, sigma=1.0, lo=16, hi=131072, n_long=4,
                     kv="bf16", seed=0) -> Workload:
    """Ragged decode, log-normal lengths clipped to [lo, hi], ``n_long`` rows at ``hi``."""
    rng = np.random.default_rng(seed)
    ctx = np.clip(np.round(np.exp(rng.normal(math.log(median), sigma, size=batch))), lo, hi)
    ctx = ctx.astype(np.int32)
    if n_long:
        ctx[rng.choice(batch, size=n_long, replace=False)] = hi
    return _decode_workload(f"long-tail-decode-{kv}", rng, ctx, 32, 8, 128, 16,
                            kv, "bf16", "bf16", seed=seed)


def mixed_prefill_decode(prior=(0, 2048, 8192, 32768), chunk=512, n_decode=128,
                         dlo=512, dhi=8192, seed=0, chunk_lens=None, n_q=32, n_kv=8, hd=128,
                         bs=16, kv="bf16") -> Workload:
    """Chunked-prefill step: prefill chunks (rows first) plus single-token decodes."""
    rng = np.random.default_rng(seed)
    prior = np.asarray(prior, np.int32)
    L = np.asarray(chunk_lens if chunk_lens is not None else [chunk] * len(prior), np.int32)
    dctx = rng.integers(dlo, dhi + 1, size=n_decode).astype(np.int32)
    ctx = np.concatenate([prior + L, dctx]).astype(np.int32)
    tables, nb = _assign_blocks(rng, ctx, bs)
    P = len(prior)
    rs = np.zeros(len(ctx), np.int32)
    rl = np.concatenate([prior, dctx - 1]).astype(np.int32)
    ns = rl.copy()
    nl = np.concatenate([L, np.ones(n_decode, np.int32)]).astype(np.int32)
    qdt = "f32" if kv == "f32" else "bf16"     # an fp32 cache takes fp32 queries and rows
    return Workload(name="mixed-prefill-decode", cache_dtype=kv, q_dtype=qdt,
                    src_dtype=qdt, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=hd,
                    block_size=bs, num_blocks=nb, context_lens=ctx, block_tables=tables,
                    q_lens=nl.copy(), res_start=rs, res_len=rl, new_start=ns, new_len=nl,
                    scale=1.0 / math.sqrt(hd), num_prefill_seqs=P, seed=seed)


CONFIGS = {
    1: worked_example,
    2: llama2_7b_decode,
    3: llama3_8b_gqa_decode,
    4: long_tail_decode,
    5: mixed_prefill_decode,
}


def small(cfg: int, seed: int = 0, kv: str = "bf16") -> Workload:
    """Reduced sizes the oracle finishes in seconds; same head shapes and block size,
    several split lengths and a ragged last block per sequence."""
    if cfg == 1:
        return worked_example()
    if cfg == 2:
        return llama2_7b_decode(batch=5, lo=17, hi=1300, seed=seed)
    if cfg == 3:
        return llama3_8b_gqa_decode(batch=7, lo=900, hi=2600, n_shared=3, seed=seed)
    if cfg == 4:
        return long_tail_decode(batch=12, median=200, sigma=1.0, lo=1, hi=5000, n_long=1,
                                kv=kv, seed=seed)
    if cfg == 5:
        return mixed_prefill_decode(prior=(0, 77, 700), chunk_lens=(64, 100, 37),
                                    n_decode=6, dlo=1, dhi=700, seed=seed)
    raise ValueError(cfg)


def full(cfg: int, seed: int = 0, kv: str = "bf16") -> Workload:
    if cfg == 4:
        return long_tail_decode(kv=kv, seed=seed)
    return CONFIGS[cfg](seed=seed) if cfg != 1 else worked_example()
