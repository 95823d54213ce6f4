"""GPU parity: slot mapping, KV append and paged decode against the oracle.

Reduced-size workloads (same head shapes and block sizes as the full
configurations, several splits and a ragged last block per sequence) are
compared in full; the full-size configurations in the launch configuration the
benchmark times are compared on sampled sequences.

Bars: integer and byte results bit-exact; fp32 outputs within 1e-5 normwise
relative error per row (max|g - r| / max|r|); bf16 / fp8- and int8-KV outputs within
2e-2 absolute AND 1e-2 normwise relative error per row.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import (blocks_of, codes, normwise_rel, oracle_decode, oracle_pools, oracle_slots)

pytestmark = pytest.mark.gpu

DECODE_CASES = [(1, "f32"), (2, "bf16"), (3, "bf16"), (4, "bf16"), (4, "fp8"), (4, "int8"),
                (5, "bf16")]


def _small(cfg, kv="bf16", seed=0):
    w = workloads.small(cfg, seed=seed, kv=kv if cfg == 4 else "bf16")
    return workloads.draw_values(w, "cpu")


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    nrm = normwise_rel(got, ref)
    if dtype == "f32":
        assert nrm.max() <= 1e-5, f"{what}: normwise {nrm.max():.3e} > 1e-5"
    else:
        err = np.abs(got - ref).max()
        assert err <= 2e-2, f"{what}: abs err {err:.3e} > 2e-2"
        assert nrm.max() <= 1e-2, f"{what}: normwise {nrm.max():.3e} > 1e-2"
    assert np.isfinite(got).all(), f"{what}: non-finite output"


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from gpu_harness import DeviceWorkload  # noqa: F401  (loads the library)
    import paged_kv_cache_74_amd as pa
    pa.lib()
    return "cuda"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_slot_mapping_bit_exact(dev, cfg):
    from gpu_harness import DeviceWorkload
    w = _small(cfg)
    dw = DeviceWorkload(w, dev)
    res = dw.append_resident().cpu().numpy()
    new = dw.append_new().cpu().numpy()
    np.testing.assert_array_equal(res, oracle_slots(w, "res"))
    np.testing.assert_array_equal(new, oracle_slots(w, "new"))


def test_worked_example_on_gpu(dev):
    """The block-size-4 example: the decode tokens land in slots 21 (A.t9) and 17 (B.t5)."""
    from gpu_harness import DeviceWorkload
    w = _small(1)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    np.testing.assert_array_equal(dw.append_new().cpu().numpy(), [21, 17])
    pk = codes(dw.k_cache, "f32")
    # free blocks 0, 1, 6 and the two unused slots of blocks 5 and 4 keep the poison
    assert (pk[[0, 1, 6]] == 0xFFC0DEAD).all()
    assert (pk[5, 2:] == 0xFFC0DEAD).all() and (pk[4, 2:] == 0xFFC0DEAD).all()


@pytest.mark.parametrize("cfg,kv", DECODE_CASES)
def test_append_pool_bit_exact(dev, cfg, kv):
    from gpu_harness import DeviceWorkload
    w = _small(cfg, kv)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    torch.cuda.synchronize()
    pk, pv = oracle_pools(w)
    np.testing.assert_array_equal(codes(dw.k_cache, w.cache_dtype), pk)
    np.testing.assert_array_equal(codes(dw.v_cache, w.cache_dtype), pv)


@pytest.mark.parametrize("split", [0, 16, 48, 1 << 20])
@pytest.mark.parametrize("cfg,kv", DECODE_CASES)
def test_decode_matches_oracle(dev, cfg, kv, split):
    from gpu_harness import DeviceWorkload, to_f64
    w = _small(cfg, kv)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    out = to_f64(dw.decode(split_tokens=split))
    pk, pv = oracle_pools(w)
    ref = oracle_decode(w, pk, pv)
    check_close(out, ref, w.q_dtype, f"cfg{cfg}/{kv}/split{split}")


@pytest.mark.parametrize("cfg,kv", [(2, "bf16"), (3, "bf16"), (4, "fp8"), (4, "int8")])
def test_decode_peaked_scores(dev, cfg, kv):
    """q scaled by 16 (exact in bf16): sharper softmax, larger dynamic range."""
    from gpu_harness import DeviceWorkload, to_f64
    w = _small(cfg, kv, seed=3)
    w.q = w.q * 16
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    out = to_f64(dw.decode())
    pk, pv = oracle_pools(w)
    check_close(out, oracle_decode(w, pk, pv), w.q_dtype, "peaked")


@pytest.mark.parametrize("cfg", [1, 3])
def test_decode_one_hot_is_exact(dev, cfg):
    """One key beats the rest by > 800: the output is that key's value, bit for bit."""
    from gpu_harness import DeviceWorkload
    w = _small(cfg)
    w.scale = 1.0
    s = int(np.argmax(w.context_lens))
    t = int(w.context_lens[s]) // 2          # a resident token of sequence s
    d = 5
    w.res_k.zero_()
    w.new_k.zero_()
    row = int(w.cu(w.res_len)[s]) + t - int(w.res_start[s])
    w.res_k[row, :, d] = 64.0
    w.q.zero_()
    w.q[s, :, d] = 64.0
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    out = dw.decode().cpu()
    want = w.res_v[row].repeat_interleave(w.group_size, dim=0)
    assert torch.equal(out[s].view(torch.int16 if cfg != 1 else torch.int32),
                       want.view(torch.int16 if cfg != 1 else torch.int32))


def test_decode_block_permutation_bit_identical(dev):
    from gpu_harness import DeviceWorkload, i32
    w = _small(3)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    base = dw.decode().clone()
    pi = torch.as_tensor(np.random.default_rng(1).permutation(w.num_blocks), device=dev)
    k2 = torch.empty_like(dw.k_cache)
    v2 = torch.empty_like(dw.v_cache)
    k2[pi] = dw.k_cache
    v2[pi] = dw.v_cache
    t = torch.as_tensor(w.block_tables, device=dev).long()
    t2 = torch.where(t >= 0, pi[t.clamp(min=0)], t).to(torch.int32).contiguous()
    dw.k_cache, dw.v_cache, dw.tables = k2, v2, t2
    again = dw.decode()
    assert torch.equal(base.view(torch.int16), again.view(torch.int16))


def test_decode_deterministic(dev):
    from gpu_harness import DeviceWorkload
    w = _small(4)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    a = dw.decode().clone()
    b = dw.decode()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_rejects_bad_arguments(dev):
    import paged_kv_cache_74_amd as pa
    from gpu_harness import DeviceWorkload
    w = _small(3)
    dw = DeviceWorkload(w, dev)
    q, tables, ctx = dw.decode_inputs()
    with pytest.raises(pa.PagedAttentionError, match="WORKSPACE"):
        pa.pa_decode(q, dw.k_cache, dw.v_cache, tables, ctx, int(w.context_lens.max()), w.scale,
                     ws=torch.empty(256, dtype=torch.uint8, device=dev))
    with pytest.raises(pa.PagedAttentionError, match="DTYPE"):
        pa.pa_decode(q.float(), dw.k_cache, dw.v_cache, tables, ctx, int(w.context_lens.max()),
                     w.scale)


# --------------------------------------------------------------------------
# full-size configurations, sampled sequences
# --------------------------------------------------------------------------

def _sample_rows(w, k=4, seed=0):
    rows = list(w.decode_rows)
    ctx = w.context_lens
    pick = {max(rows, key=lambda s: ctx[s]), min(rows, key=lambda s: ctx[s])}
    if w.shared_prefix_seqs:
        pick.add(w.shared_prefix_seqs[-1])
    rng = np.random.default_rng(seed)
    while len(pick) < k + 2:
        pick.add(int(rng.choice(rows)))
    return sorted(pick)


@pytest.mark.parametrize("cfg,kv", [(2, "bf16"), (3, "bf16"), (4, "bf16"), (4, "fp8"), (4, "int8"),
                                    (5, "bf16")])
def test_full_size_decode_sampled(dev, cfg, kv):
    from gpu_harness import DeviceWorkload, to_f64
    print(f"full-size decode cfg{cfg} {kv}", flush=True)
    w = workloads.full(cfg, kv=kv)
    workloads.draw_values(w, dev)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    out = dw.decode()
    torch.cuda.synchronize()
    rows = _sample_rows(w)
    pk, pv = oracle_pools(w, seqs=rows)
    blocks = torch.as_tensor(blocks_of(w, rows), device=dev)
    np.testing.assert_array_equal(codes(dw.k_cache.index_select(0, blocks), w.cache_dtype),
                                  pk[blocks.cpu().numpy()])
    np.testing.assert_array_equal(codes(dw.v_cache.index_select(0, blocks), w.cache_dtype),
                                  pv[blocks.cpu().numpy()])
    ref = oracle_decode(w, pk, pv, rows=rows)
    P = w.num_prefill_seqs
    got = to_f64(out)[[r - P for r in rows]]
    check_close(got, ref, w.q_dtype, f"full cfg{cfg}/{kv}")


def test_decode_phases_equal_one_call(dev):
    """pa_decode_partials + pa_decode_merge == pa_decode, bit for bit."""
    import paged_kv_cache_74_amd as pa
    from gpu_harness import DeviceWorkload
    w = _small(4, "fp8")
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    one = dw.decode().clone()
    q, tables, ctx = dw.decode_inputs()
    maxc = int(w.context_lens.max())
    ws = pa.workspace(pa.pa_decode_workspace_bytes(q.shape[0], w.n_q_heads, w.n_kv_heads,
                                                   w.head_dim, maxc), dev)
    pa.pa_decode_partials(q, dw.k_cache, dw.v_cache, tables, ctx, maxc, w.scale, ws, w.k_scale)
    two = pa.pa_decode_merge(torch.empty_like(q), ctx, w.n_kv_heads, maxc, ws, w.v_scale)
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


def test_decode_workspace_reuse(dev):
    """One workspace reused across calls with different split sizes and a two-phase call:
    nothing a call leaves in it changes the next call's result."""
    import paged_kv_cache_74_amd as pa
    from gpu_harness import DeviceWorkload
    w = _small(4)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    q, tables, ctx = dw.decode_inputs()
    maxc = int(w.context_lens.max())
    ws = pa.workspace(pa.pa_decode_workspace_bytes(q.shape[0], w.n_q_heads, w.n_kv_heads,
                                                   w.head_dim, maxc, 16), dev)
    args = (q, dw.k_cache, dw.v_cache, tables, ctx, maxc, w.scale, w.k_scale, w.v_scale)
    r0 = pa.pa_decode(*args, ws=ws, split_tokens=16).clone()
    pa.pa_decode_partials(q, dw.k_cache, dw.v_cache, tables, ctx, maxc, w.scale, ws, w.k_scale,
                          split_tokens=16)
    r1 = pa.pa_decode_merge(torch.empty_like(q), ctx, w.n_kv_heads, maxc, ws, w.v_scale,
                            split_tokens=16)
    r2 = pa.pa_decode(*args, ws=ws, split_tokens=16).clone()
    r3 = pa.pa_decode(*args, ws=ws, split_tokens=48).clone()
    r4 = pa.pa_decode(*args, ws=ws, split_tokens=16)
    for r in (r1, r2, r4):
        assert torch.equal(r0.view(torch.int16), r.view(torch.int16))
    from gpu_harness import to_f64
    pk, pv = oracle_pools(w)
    check_close(to_f64(r3), oracle_decode(w, pk, pv), w.q_dtype,
                "split 48 after split 16 on one workspace")


# (n_q, n_kv, head_dim, block_size) for the bf16 and 8-bit caches: every group
# size, both head dims, block sizes that take the matrix-core kernel (>= 16) and
# one that takes the vector kernel; int8 on 8 x 2 x 64 loads per head, the other
# matrix-core shapes stage their loads through LDS (bf16 reading V from the stage);
# one KV head per workgroup: bf16 128 stages, bf16 64 and the 8-bit caches load per head
SHAPES_8BIT = [(8, 8, 128, 16), (8, 4, 64, 32), (16, 4, 128, 16), (32, 4, 64, 64),
               (16, 2, 128, 8), (8, 2, 64, 16), (32, 4, 128, 32), (8, 1, 128, 16),
               (4, 1, 64, 16)]


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("nq,nkv,hd,bs", SHAPES_8BIT)
def test_decode_shapes(dev, kv, nq, nkv, hd, bs):
    from gpu_harness import DeviceWorkload, to_f64
    rng = np.random.default_rng(nq * 7 + hd + bs)
    ctx = rng.integers(1, 900, 9).astype(np.int32)
    ctx[0] = 1
    w = workloads._decode_workload("shapes", rng, ctx, nq, nkv, hd, bs, kv, "bf16", "bf16",
                                   seed=4)
    workloads.draw_values(w, "cpu")
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    for split in (0, 48):
        got = to_f64(dw.decode(split_tokens=split))
        pk, pv = oracle_pools(w)
        check_close(got, oracle_decode(w, pk, pv), "bf16", f"{kv} {nq}/{nkv}/{hd}/bs{bs} split {split}")
