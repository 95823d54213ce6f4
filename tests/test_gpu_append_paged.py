"""GPU parity of pa_kv_append_paged / pa_kv_append_int4_paged (slot map and append in one launch).

Bars: bit-exact.  The pools, value scales and returned slots must equal the
oracle's on the reduced-size workloads, and equal the two-call path
(pa_slot_mapping, then pa_kv_append[_int4]) on ragged edge cases: empty
segments, positions past the table row, negative table entries, negative
start positions, and a grid hint far below the longest segment.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import codes, oracle_pools, oracle_pools_int4, oracle_slots

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import paged_kv_cache_74_amd as pa
    pa.lib()
    return "cuda"


@pytest.mark.parametrize("cfg,kv", [(1, "f32"), (2, "bf16"), (3, "bf16"), (4, "fp8"), (4, "int8"),
                                    (5, "bf16"), (3, "int4"), (5, "int4")])
def test_paged_append_matches_oracle(dev, cfg, kv):
    from gpu_harness import DeviceWorkload
    w = workloads.small(cfg, kv=kv if cfg == 4 else "bf16")
    if kv == "int4":
        w.cache_dtype = "int4"
    workloads.draw_values(w, "cpu")
    dw = DeviceWorkload(w, dev, paged_append=True)
    res = dw.append_resident().cpu().numpy()
    new = dw.append_new().cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(res, oracle_slots(w, "res"))
    np.testing.assert_array_equal(new, oracle_slots(w, "new"))
    if kv == "int4":
        pk, pv, ps = oracle_pools_int4(w)
        np.testing.assert_array_equal(dw.k_cache.cpu().numpy(), pk)
        np.testing.assert_array_equal(dw.v_cache.cpu().numpy(), pv)
        np.testing.assert_array_equal(dw.v_scales.cpu().numpy().view(np.uint32),
                                      ps.view(np.uint32))
    else:
        pk, pv = oracle_pools(w)
        np.testing.assert_array_equal(codes(dw.k_cache, w.cache_dtype), pk)
        np.testing.assert_array_equal(codes(dw.v_cache, w.cache_dtype), pv)


def _edge_batch(rng, nb, bs, max_blocks):
    """Ragged segments with every edge the map has."""
    lens = [0, 1, 37, 0, 200, 1, 5, 64, 3]
    start = [0, 10, 3, 5, 17, 0, -2, bs * max_blocks - 30, 0]   # one runs past the row
    S = len(lens)
    # distinct blocks, so no two tokens share a slot
    tables = rng.permutation(nb)[:S * max_blocks].reshape(S, max_blocks).astype(np.int32)
    tables[2, 1] = -1                                  # a hole in a row
    tables[8, :] = -1                                  # a row with no blocks at all
    cu = np.zeros(S + 1, np.int32)
    np.cumsum(lens, out=cu[1:])
    return tables, cu, np.array(start, np.int32), int(cu[-1]), max(lens)


@pytest.mark.parametrize("kv,src", [("bf16", "bf16"), ("f32", "f32"), ("fp8", "bf16"),
                                    ("int8", "f32"), ("int4", "bf16"), ("int4", "f32")])
@pytest.mark.parametrize("hint", [1, None])
def test_paged_append_equals_two_calls(dev, kv, src, hint):
    import paged_kv_cache_74_amd as pa
    from workloads import INT4_SCALE_POISON
    rng = np.random.default_rng(11)
    nb, bs, nkv, hd, max_blocks = 200, 16, 4, 128, 20
    tables, cu, start, T, longest = _edge_batch(rng, nb, bs, max_blocks)
    hint = longest if hint is None else hint
    tdt = torch.bfloat16 if src == "bf16" else torch.float32
    k = (torch.randn(T, nkv, hd, generator=torch.Generator().manual_seed(1)) * 2).to(tdt).to(dev)
    v = (torch.randn(T, nkv, hd, generator=torch.Generator().manual_seed(2)) * 2).to(tdt).to(dev)
    g_tab, g_cu, g_start = (torch.as_tensor(x, device=dev) for x in (tables, cu, start))
    if kv == "int4":
        pool = lambda: torch.full((nb, bs, nkv, hd // 2), 0x77, dtype=torch.uint8, device=dev)
        scl = lambda: torch.full((nb, nkv, bs), int(INT4_SCALE_POISON) - (1 << 32),
                                 dtype=torch.int32, device=dev).view(torch.float32)
        ks = torch.as_tensor(rng.uniform(0.05, 2.0, (nkv, hd)).astype(np.float32), device=dev)
        a = (pool(), pool(), scl())
        b = (pool(), pool(), scl())
        slots_a = pa.pa_slot_mapping(g_tab, g_cu, g_start, bs, T)
        pa.pa_kv_append_int4(*a, k, v, slots_a, ks)
        slots_b = torch.full((T,), -7, dtype=torch.int64, device=dev)
        pa.pa_kv_append_int4_paged(*b, k, v, g_tab, g_cu, g_start, hint, ks, slot_mapping=slots_b)
        c = (pool(), pool(), scl())
        pa.pa_kv_append_int4_paged(*c, k, v, g_tab, g_cu, g_start, hint, ks)   # no slot output
    else:
        cdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8,
               "int8": torch.int8}[kv]
        fill = 0x5A if kv in ("fp8", "int8") else float("nan")   # poison: untouched bytes stay
        pool = lambda: torch.full((nb, bs, nkv, hd), fill, dtype=cdt, device=dev)
        sc = (0.37, 1.9) if kv in ("fp8", "int8") else (1.0, 1.0)
        a = (pool(), pool())
        b = (pool(), pool())
        slots_a = pa.pa_slot_mapping(g_tab, g_cu, g_start, bs, T)
        pa.pa_kv_append(*a, k, v, slots_a, *sc)
        slots_b = torch.full((T,), -7, dtype=torch.int64, device=dev)
        pa.pa_kv_append_paged(*b, k, v, g_tab, g_cu, g_start, hint, slot_mapping=slots_b,
                              k_scale=sc[0], v_scale=sc[1])
        c = (pool(), pool())
        pa.pa_kv_append_paged(*c, k, v, g_tab, g_cu, g_start, hint, k_scale=sc[0], v_scale=sc[1])
    torch.cuda.synchronize()
    sa = slots_a.cpu().numpy()
    assert (sa == -1).any() and (sa >= 0).any()        # the batch does exercise skipped tokens
    np.testing.assert_array_equal(slots_b.cpu().numpy(), sa)
    for x, y, z in zip(a, b, c):
        xb = x.view(torch.uint8).cpu().numpy()
        np.testing.assert_array_equal(y.view(torch.uint8).cpu().numpy(), xb)
        np.testing.assert_array_equal(z.view(torch.uint8).cpu().numpy(), xb)
