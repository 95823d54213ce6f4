"""pa_decode_no_alloc (the decode entry point that allocates nothing) against pa_decode.

Two calls in a row through the C ABI, the second with a smaller input (fewer
sequences, shorter contexts) than the first, so the second reads a scratch the
first left full of its own partials.  Each output must be bit-identical to
pa_decode's on the same inputs (both run the same kernels), and within the
oracle's bar (2e-2 absolute and 1e-2 normwise per row for bf16).
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import normwise_rel, oracle_decode, oracle_pools

pytestmark = pytest.mark.gpu


def _check(w, dev):
    import paged_kv_cache_74_amd as pa
    from gpu_harness import DeviceWorkload, to_f64
    print(f"no-alloc decode: {w.name}, {w.num_seqs} seqs, max ctx {int(w.context_lens.max())}",
          flush=True)
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    dw.append_new()
    q, tables, ctx = dw.decode_inputs()
    maxc = int(w.context_lens.max())
    ref = pa.pa_decode(q, dw.k_cache, dw.v_cache, tables, ctx, maxc, w.scale, w.k_scale,
                       w.v_scale)
    out = torch.full_like(q, float("nan"))
    pa.pa_decode_no_alloc(q, dw.k_cache, dw.v_cache, tables, ctx, maxc, w.scale, out,
                          w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "differs from pa_decode"
    pk, pv = oracle_pools(w)
    got, exp = to_f64(out), oracle_decode(w, pk, pv)
    assert np.isfinite(got).all()
    assert np.abs(got - exp).max() <= 2e-2
    assert normwise_rel(got, exp).max() <= 1e-2


def test_no_alloc_decode_twice_second_smaller():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    dev = "cuda"
    first = workloads.draw_values(workloads.small(3), "cpu")                  # 7 seqs, ctx 900..2600
    second = workloads.draw_values(
        workloads.llama3_8b_gqa_decode(batch=3, lo=40, hi=300, n_shared=0, prefix_tokens=16,
                                       seed=5), "cpu")
    assert second.num_seqs < first.num_seqs and second.context_lens.max() < first.context_lens.min()
    _check(first, dev)
    _check(second, dev)


def test_no_alloc_rejects_what_does_not_fit():
    """Sizes whose partials exceed the scratch return PA_ERR_WORKSPACE, before any launch."""
    import paged_kv_cache_74_amd as pa
    L = pa.lib()
    B = 1 << 16
    need = pa.pa_decode_workspace_bytes(B, 32, 8, 128, 4096, 0)
    assert need > pa.PA_NO_ALLOC_SCRATCH_BYTES
    st = L.pa_decode_no_alloc(None, None, pa.PA_BF16, None, None, pa.PA_BF16, 8, 16, 8, 128, 4,
                              None, 256, None, B, 4096, 0.1, 1.0, 1.0, 0, None)
    assert st == 5   # PA_ERR_WORKSPACE
