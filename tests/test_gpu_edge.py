"""GPU edge cases through the C-ABI, against the oracle.  Decode: sequences with
an empty context beside full ones (their output rows must be exactly zero), a
batch whose contexts are all empty, the largest block size (256 tokens), and the
appending decode over empty contexts (no slot, slot -1).  Prefill: chunks of 0
and 1 queries beside longer ones, causal or not, with and without the decode path
for the rows of length 1.

Bars as elsewhere: bf16 / 8-bit outputs within 2e-2 absolute and 1e-2 normwise
relative error per row; a zero reference row must come back exactly zero (the
normwise check divides by 1e-300 there).
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import oracle_decode, oracle_decode_int4, oracle_pools, oracle_pools_int4
from test_gpu_decode import check_close

pytestmark = pytest.mark.gpu

CTX = [0, 5, 0, 700, 1, 0, 33, 290]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import paged_kv_cache_74_amd as pa
    pa.lib()
    return "cuda"


def _built(dev, ctx, kv, nq, nkv, hd, bs, seed=2, spare=0):
    from gpu_harness import DeviceWorkload
    rng = np.random.default_rng(seed)
    w = workloads._decode_workload("edge", rng, np.asarray(ctx, np.int32), nq, nkv, hd, bs, kv,
                                   "bf16", "bf16", spare=spare, seed=seed)
    workloads.draw_values(w, "cpu")
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    return w, dw


def _reference(w):
    if w.cache_dtype == "int4":
        pk, pv, ps = oracle_pools_int4(w)
        return oracle_decode_int4(w, pk, pv, ps)
    pk, pv = oracle_pools(w)
    return oracle_decode(w, pk, pv)


# (cache, n_q, n_kv, head_dim, block_size): the staged matrix-core kernel (bf16,
# fp8, int8), per-head loads (int4), the vector kernel (blocks of 8) and blocks
# of 256 tokens
EDGE_SHAPES = [("bf16", 32, 8, 128, 16), ("fp8", 32, 8, 128, 16), ("int8", 16, 4, 128, 32),
               ("int4", 32, 8, 128, 16), ("bf16", 8, 2, 64, 8), ("bf16", 8, 8, 128, 256),
               ("int8", 16, 4, 64, 256)]


@pytest.mark.parametrize("kv,nq,nkv,hd,bs", EDGE_SHAPES)
def test_decode_empty_contexts_beside_full_ones(dev, kv, nq, nkv, hd, bs):
    from gpu_harness import to_f64
    print(f"edge decode {kv} {nq}/{nkv}/{hd}/bs{bs}", flush=True)
    w, dw = _built(dev, CTX, kv, nq, nkv, hd, bs)
    ref = _reference(w)
    for split in (0, 16):
        got = to_f64(dw.decode(split_tokens=split))
        empty = np.asarray(CTX) == 0
        assert (got[empty] == 0).all(), f"{kv} split {split}: rows of empty contexts not zero"
        check_close(got, ref, "bf16", f"{kv} {nq}/{nkv}/{hd}/bs{bs} split {split}")


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_decode_all_contexts_empty(dev, kv):
    """Every context empty: no unit of work anywhere, every output row zero.  (The
    pools still hold a few blocks: the call takes real pool pointers.)"""
    from gpu_harness import to_f64
    w, dw = _built(dev, [0] * 6, kv, 32, 8, 128, 16, spare=4)
    out = torch.full_like(dw.q, float("nan"))
    got = to_f64(dw.decode(out=out))
    assert (got == 0).all()


def test_decode_append_over_empty_contexts(dev):
    """The appending decode on a batch with empty contexts: those sequences append
    nothing (slot -1) and their rows are zero; the others match the separate
    append + decode bit for bit."""
    import paged_kv_cache_74_amd as pa
    from gpu_harness import DeviceWorkload, i32, to_f64
    w, dw = _built(dev, CTX, "bf16", 32, 8, 128, 16)
    ref_out = to_f64(dw.decode())
    # a second pool with the resident tokens only; the call appends the new ones
    two = DeviceWorkload(w, dev)
    two.append_resident()
    ctx = np.asarray(CTX)
    B = len(CTX)
    new_k = torch.zeros((B,) + tuple(w.new_k.shape[1:]), dtype=w.new_k.dtype)
    new_v = torch.zeros_like(new_k)
    rows = np.flatnonzero(ctx > 0)
    new_k[rows] = w.new_k
    new_v[rows] = w.new_v
    slots = torch.full((B,), 7, dtype=torch.int64, device=dev)
    maxc = int(ctx.max())
    out = pa.pa_decode_append(two.q, two.k_cache, two.v_cache, new_k.to(dev), new_v.to(dev),
                              two.tables, two.ctx, maxc, w.scale, 1.0, 1.0, slot_mapping=slots)
    got = to_f64(out)
    s = slots.cpu().numpy()
    assert (s[ctx == 0] == -1).all()
    assert (s[ctx > 0] >= 0).all()
    assert (got[ctx == 0] == 0).all()
    assert np.array_equal(got, ref_out)
    assert torch.equal(two.k_cache.view(torch.int16), dw.k_cache.view(torch.int16))
    assert torch.equal(two.v_cache.view(torch.int16), dw.v_cache.view(torch.int16))


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("bs", [16, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_empty_and_single_query_chunks(dev, kv, bs, causal):
    """Chunks of 0 queries (a sequence with no rows in the batch), 1 query (run on the
    decode path when blocks hold 16 tokens or more) and a few queries, over prior
    contexts of 0 to 400 tokens, in one pa_prefill_chunk call."""
    from gpu_harness import DeviceWorkload, prefill, to_f64
    from helpers import oracle_prefill
    print(f"edge prefill {kv} bs{bs} causal={causal}", flush=True)
    w = workloads.mixed_prefill_decode(prior=(10, 0, 50, 400, 64), chunk_lens=(0, 7, 0, 1, 33),
                                       n_decode=3, dlo=1, dhi=90, seed=5, n_q=16, n_kv=4, hd=128,
                                       bs=bs, kv=kv)
    workloads.draw_values(w, "cpu")
    w.causal = causal
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    got = to_f64(prefill(dw))
    pk, pv = oracle_pools(w)
    check_close(got, oracle_prefill(w, pk, pv), "bf16", f"prefill edge {kv} bs{bs} causal={causal}")
