"""Pins of the oracle's INT4 KV cache (per-channel K scales, per-token V scales).

The format is the reading stated in oracle/codecs.py: symmetric 4-bit codes in
[-7, 7], two per byte in sign-magnitude nibbles (element 2i low); keys use
one scale per (KV head, channel), values one scale per (token, KV head) equal
to the row's amax / 7.  Checked against hand-derived bytes, torch's rounding,
the quantisation error bound and an attention computed from independently
unpacked values.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import codecs, paged


def test_int4_pack_bytes_by_hand():
    # low nibble = element 0; a negative code sets the nibble's bit 3
    assert codecs.int4_pack(np.array([1, -1])).tolist() == [0x91]
    assert codecs.int4_pack(np.array([-7, 7])).tolist() == [0x7F]
    assert codecs.int4_pack(np.array([0, -3])).tolist() == [0xB0]
    assert codecs.int4_pack(np.array([7, 0, 2, -2])).tolist() == [0x07, 0xA2]


def test_int4_every_code_pair_round_trips():
    c = np.arange(-7, 8)
    a, b = np.meshgrid(c, c, indexing="ij")
    pairs = np.stack([a.ravel(), b.ravel()], axis=-1)
    assert np.array_equal(codecs.int4_unpack(codecs.int4_pack(pairs)), pairs.astype(np.float64))


def test_int4_negative_zero_nibble_is_zero():
    assert codecs.int4_unpack(np.array([0x88, 0x80, 0x08], np.uint8)).tolist() == [0, 0, 0, 0, 0, 0]


def test_int4_encode_ties_to_even_and_saturation():
    x = np.array([2.5, 3.5, -0.5, -2.5, 6.5, 7.5, 7.49, 100.0, -np.inf, np.inf, np.nan, -6.5],
                 np.float32)
    assert codecs.int4_encode(x).tolist() == [2, 4, 0, -2, 6, 7, 7, 7, -7, 7, 0, -6]


def test_int4_encode_matches_torch_round_and_clamp():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 5).astype(np.float32)
    x[::97] = np.rint(x[::97]) + 0.5                      # exact ties
    t = torch.from_numpy(x).round().clamp(-7, 7).to(torch.int8).numpy()
    assert np.array_equal(codecs.int4_encode(x), t)


def test_int4_token_scale_bounds_the_error():
    """Per-token V: the row's largest magnitude maps to +-7, every element is
    within half a step (sigma / 2) of its dequantised value, and scaling one row
    leaves the codes of the others unchanged."""
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((64, 2, 128)) * rng.uniform(0.01, 50, (64, 2, 1))).astype(np.float32)
    src = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    k = np.zeros_like(src)
    _, pv, sig = paged.encode_int4_tokens(k, src, "bf16", np.ones((2, 128), np.float32))
    x = codecs.bf16_decode(src)
    codes = codecs.int4_unpack(pv)
    i = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(codes, i[..., None], -1)[..., 0]
    assert np.array_equal(np.abs(top), np.full(top.shape, 7.0))
    assert np.array_equal(np.sign(top), np.sign(np.take_along_axis(x, i[..., None], -1)[..., 0]))
    s = sig.astype(np.float64)[..., None]
    assert np.all(np.abs(x - codes * s) <= s / 2 * (1 + 2.0 ** -20))
    src2 = src.copy()
    src2[5] = torch.from_numpy(v[5] * 1000).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, pv2, sig2 = paged.encode_int4_tokens(k, src2, "bf16", np.ones((2, 128), np.float32))
    keep = np.arange(64) != 5
    assert np.array_equal(pv2[keep], pv[keep]) and np.array_equal(sig2[keep], sig[keep])


def test_int4_token_scale_edge_rows():
    rows = np.zeros((3, 8), np.float32)
    rows[1] = [1, -2, np.nan, 3, 0, 0, 0, -7]              # NaN ignored in amax, encodes 0
    rows[2] = [0, 0, 0, 0, 0, 0, 0, -0.0]
    src = rows.view(np.uint32)
    _, pv, sig = paged.encode_int4_tokens(np.zeros_like(src), src, "f32",
                                          np.ones(8, np.float32))
    assert sig.tolist() == [0.0, 1.0, 0.0]
    assert codecs.int4_unpack(pv).tolist() == [[0] * 8, [1, -2, 0, 3, 0, 0, 0, -7], [0] * 8]


def test_int4_key_channel_scales():
    """Per-channel K: channel d's codes are k / s_d rounded (within s_d / 2 unless
    saturated), and changing one channel's scale changes only that channel."""
    rng = np.random.default_rng(5)
    s = rng.uniform(0.05, 2.0, (2, 64)).astype(np.float32)
    x = (rng.uniform(-7.4, 7.4, (100, 2, 64)) * s[None]).astype(np.float32)
    src = x.view(np.uint32)
    pk, _, _ = paged.encode_int4_tokens(src, src, "f32", s)
    codes = codecs.int4_unpack(pk)
    sd = s.astype(np.float64)[None]
    assert np.all(np.abs(x - codes * sd) <= sd / 2 * (1 + 2.0 ** -20))
    s2 = s.copy()
    s2[1, 7] *= 3
    pk2, _, _ = paged.encode_int4_tokens(src, src, "f32", s2)
    c2 = codecs.int4_unpack(pk2)
    mask = np.ones((2, 64), bool)
    mask[1, 7] = False
    assert np.array_equal(c2[:, mask], codes[:, mask])
    assert not np.array_equal(c2[:, 1, 7], codes[:, 1, 7])


def _tiny_int4_cache(rng, nb=12, bs=4, nkv=2, hd=16, B=3):
    ctx = rng.integers(1, 14, B)
    perm = rng.permutation(nb)
    nblk = -(-ctx // bs)
    tables = -np.ones((B, nblk.max()), np.int32)
    used = 0
    for s in range(B):
        tables[s, :nblk[s]] = perm[used:used + nblk[s]]
        used += nblk[s]
    pk = np.full((nb, bs, nkv, hd // 2), 0x77, np.uint8)
    pv = np.full((nb, bs, nkv, hd // 2), 0x77, np.uint8)
    ps = np.full((nb, nkv, bs), np.nan, np.float32)
    ks = rng.uniform(0.1, 1.0, (nkv, hd)).astype(np.float32)
    for s in range(B):
        n = int(ctx[s])
        k = torch.from_numpy(rng.standard_normal((n, nkv, hd)).astype(np.float32)).to(torch.bfloat16)
        v = torch.from_numpy(rng.standard_normal((n, nkv, hd)).astype(np.float32)).to(torch.bfloat16)
        kc = k.view(torch.int16).numpy().view(np.uint16)
        vc = v.view(torch.int16).numpy().view(np.uint16)
        slots = paged.slot_mapping(tables[s:s + 1], np.array([0]), np.array([n]), bs)
        paged.kv_append_int4(pk, pv, ps, kc, vc, slots, bs, "bf16", ks)
    return pk, pv, ps, ks, tables, ctx


def test_int4_decode_equals_attention_over_unpacked_values():
    """decode_int4 against attention computed from values unpacked nibble by
    nibble in plain Python, token by token through the block table."""
    rng = np.random.default_rng(6)
    nkv, hd, G, bs = 2, 16, 2, 4
    pk, pv, ps, ks, tables, ctx = _tiny_int4_cache(rng, bs=bs, nkv=nkv, hd=hd)
    B = len(ctx)
    q = torch.from_numpy(rng.standard_normal((B, nkv * G, hd)).astype(np.float32)).to(torch.bfloat16)
    qc = q.view(torch.int16).numpy().view(np.uint16)
    got = paged.decode_int4(qc, "bf16", pk, pv, ps, ks, tables, ctx, bs, G, 0.25)

    def nib(byte, hi):
        n = (int(byte) >> 4) & 0xF if hi else int(byte) & 0xF
        return -(n & 7) if n & 8 else (n & 7)

    qf = codecs.bf16_decode(qc)
    for s in range(B):
        for h in range(nkv * G):
            g = h // G
            K = np.zeros((ctx[s], hd))
            V = np.zeros((ctx[s], hd))
            for p in range(ctx[s]):
                blk, off = tables[s, p // bs], p % bs
                for d in range(hd):
                    K[p, d] = nib(pk[blk, off, g, d // 2], d % 2) * float(ks[g, d])
                    V[p, d] = nib(pv[blk, off, g, d // 2], d % 2) * float(ps[blk, g, off])
            sc = 0.25 * (K @ qf[s, h])
            w = np.exp(sc - sc.max())
            ref = (w @ V) / w.sum()
            assert np.allclose(got[s, h], ref, rtol=1e-12, atol=1e-12)


def test_int4_decode_invariant_under_block_relabelling():
    rng = np.random.default_rng(7)
    nkv, hd, G, bs = 2, 16, 1, 4
    pk, pv, ps, ks, tables, ctx = _tiny_int4_cache(rng, bs=bs, nkv=nkv, hd=hd)
    B = len(ctx)
    q = torch.from_numpy(rng.standard_normal((B, nkv * G, hd)).astype(np.float32)).to(torch.bfloat16)
    qc = q.view(torch.int16).numpy().view(np.uint16)
    a = paged.decode_int4(qc, "bf16", pk, pv, ps, ks, tables, ctx, bs, G, 0.3)
    perm = rng.permutation(pk.shape[0])                   # new id of block b is perm[b]
    inv = np.argsort(perm)
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    b = paged.decode_int4(qc, "bf16", pk[inv], pv[inv], ps[inv], ks, t2, ctx, bs, G, 0.3)
    assert np.array_equal(a, b)


def test_int4_prefill_rows_match_decode_and_causality():
    """prefill_chunk_int4: a chunk's last query equals decode_int4 of the sequence,
    each earlier query equals decode_int4 over the cache truncated at its position,
    and the non-causal chunk lets every query see every key."""
    rng = np.random.default_rng(8)
    nkv, hd, G, bs = 2, 16, 2, 4
    pk, pv, ps, ks, tables, ctx = _tiny_int4_cache(rng, bs=bs, nkv=nkv, hd=hd)
    B = len(ctx)
    L = np.minimum(ctx, np.array([3, 1, 5])[:B])
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    q = torch.from_numpy(rng.standard_normal((int(cu[-1]), nkv * G, hd)).astype(np.float32))
    qc = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = paged.prefill_chunk_int4(qc, "bf16", cu, pk, pv, ps, ks, tables, ctx, bs, G, 0.3)
    for s in range(B):
        for i in range(int(L[s])):
            T = int(ctx[s]) - int(L[s]) + i + 1       # keys visible to query i
            qd = np.zeros((B, nkv * G, hd), np.uint16)
            qd[s] = qc[cu[s] + i]
            ref = paged.decode_int4(qd, "bf16", pk, pv, ps, ks, tables,
                                    np.where(np.arange(B) == s, T, ctx), bs, G, 0.3, rows=[s])
            assert np.allclose(got[cu[s] + i], ref[0], rtol=1e-12, atol=1e-12)
    full = paged.prefill_chunk_int4(qc, "bf16", cu, pk, pv, ps, ks, tables, ctx, bs, G, 0.3,
                                    causal=False)
    for s in range(B):
        qd = np.zeros((B, nkv * G, hd), np.uint16)
        qd[s] = qc[cu[s]]
        ref = paged.decode_int4(qd, "bf16", pk, pv, ps, ks, tables, ctx, bs, G, 0.3, rows=[s])
        assert np.allclose(full[cu[s]], ref[0], rtol=1e-12, atol=1e-12)
