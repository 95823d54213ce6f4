"""pa_decode_append (the step's append and attention in one call) against the two
calls it replaces and against the oracle.

For every case the same resident tokens are appended to two pairs of pools; one
pair then takes pa_kv_append_paged (one token per sequence at its last position)
and pa_decode, the other pa_decode_append.  The pools and slots must be
bit-identical, and so must the outputs (the same split, the same arithmetic on
the same codes); the output must also meet the oracle's bar.  Cases cover the
staged split kernel (append inside the attention launch: bf16, fp8, int8 with
blocks of 16 tokens or more) and the paths that append in a launch of their own
(fp32 caches, blocks of fewer than 16 tokens).
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import oracle_decode, oracle_pools
from test_gpu_decode import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import paged_kv_cache_74_amd as pa
    pa.lib()
    return "cuda"


def _compare(w, dev, split_tokens=0, partials=False):
    import paged_kv_cache_74_amd as pa
    from gpu_harness import DeviceWorkload, i32, to_f64
    print(f"decode_append {w.name} {w.cache_dtype} nq={w.n_q_heads} nkv={w.n_kv_heads} "
          f"hd={w.head_dim} bs={w.block_size} B={w.num_seqs}", flush=True)
    assert (w.new_len == 1).all() and np.array_equal(w.new_start, w.context_lens - 1)
    two = DeviceWorkload(w, dev, paged_append=True)
    two.append_resident()
    slots_two = two.append_new()
    ref = two.decode(split_tokens=split_tokens)
    one = DeviceWorkload(w, dev)
    one.append_resident()
    slots_one = torch.full((w.num_seqs,), -7, dtype=torch.int64, device=dev)
    maxc = int(w.context_lens.max())
    kn, vn = w.new_k.to(dev), w.new_v.to(dev)
    if partials:
        ws = pa.workspace(pa.pa_decode_workspace_bytes(w.num_seqs, w.n_q_heads, w.n_kv_heads,
                                                       w.head_dim, maxc, split_tokens), dev)
        pa.pa_decode_append_partials(one.q, one.k_cache, one.v_cache, kn, vn, one.tables,
                                     one.ctx, maxc, w.scale, ws, w.k_scale, w.v_scale,
                                     split_tokens, slot_mapping=slots_one)
        got = pa.pa_decode_merge(torch.empty_like(one.q), one.ctx, w.n_kv_heads, maxc, ws,
                                 w.v_scale if w.cache_dtype in ("fp8", "int8") else 1.0,
                                 split_tokens)
    else:
        got = pa.pa_decode_append(one.q, one.k_cache, one.v_cache, kn, vn, one.tables, one.ctx,
                                  maxc, w.scale, w.k_scale, w.v_scale, split_tokens=split_tokens,
                                  slot_mapping=slots_one)
    torch.cuda.synchronize()
    assert torch.equal(slots_one, slots_two), "slots differ from pa_kv_append_paged"
    for a, b, name in ((one.k_cache, two.k_cache, "K"), (one.v_cache, two.v_cache, "V")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} pool differs"
    ib = torch.int32 if w.q_dtype == "f32" else torch.int16
    assert torch.equal(got.view(ib), ref.view(ib)), "output differs from append + decode"
    pk, pv = oracle_pools(w)
    check_close(to_f64(got), oracle_decode(w, pk, pv), w.q_dtype, f"decode_append {w.name}")


@pytest.mark.parametrize("cfg,kv", [(1, "f32"), (2, "bf16"), (3, "bf16"), (4, "bf16"),
                                    (4, "fp8"), (4, "int8")])
def test_decode_append_small_configs(dev, cfg, kv):
    w = workloads.draw_values(workloads.small(cfg, kv=kv), "cpu")
    _compare(w, dev)


@pytest.mark.parametrize("split", [16, 48])
def test_decode_append_partials_and_splits(dev, split):
    w = workloads.draw_values(workloads.small(3), "cpu")
    _compare(w, dev, split_tokens=split, partials=True)


# (n_q, n_kv, head_dim, block_size, cache): every group size, both head dims, blocks
# below 16 (the append in a launch of its own) and above
SHAPES = [(8, 8, 128, 16, "bf16"), (8, 4, 64, 32, "fp8"), (16, 2, 128, 8, "bf16"),
          (32, 4, 64, 64, "int8"), (8, 1, 128, 16, "bf16"), (16, 8, 64, 16, "fp8"),
          (4, 4, 64, 4, "int8")]


@pytest.mark.parametrize("nq,nkv,hd,bs,kv", SHAPES)
def test_decode_append_shapes(dev, nq, nkv, hd, bs, kv):
    rng = np.random.default_rng(11)
    ctx = rng.integers(1, 400, size=6).astype(np.int32)
    ctx[0] = 1                                   # the new token is the whole context
    ctx[1] = 16 * 3                              # it ends a step exactly
    w = workloads._decode_workload("append-shapes", rng, ctx, nq, nkv, hd, bs, kv, "bf16",
                                   "bf16", seed=11)
    workloads.draw_values(w, "cpu")
    _compare(w, dev)


def test_decode_append_fp32_sources_into_8bit_caches(dev):
    """fp32 rows encoded into an fp8 cache, as pa_kv_append encodes them."""
    rng = np.random.default_rng(12)
    ctx = rng.integers(1, 300, size=5).astype(np.int32)
    w = workloads._decode_workload("append-f32src", rng, ctx, 16, 4, 128, 16, "fp8", "bf16",
                                   "f32", seed=12)
    workloads.draw_values(w, "cpu")
    _compare(w, dev)
