"""Every fp32 bit pattern through the append encoders, against the oracle.

pa_kv_append with an fp32 source and an FP8_E4M3 or INT8 cache encodes each
element as e4m3_satfinite_rne(x * (1 / scale)) or clamp(rint(x * (1 / scale)))
(include/pa.h).  With scale 1 the product is x itself, so the 2^32 inputs below
are every input the encoder can see.  The sweep runs in 2^28-pattern chunks
(one test case each): the GPU appends a chunk as K and V rows into token-major
pools (slot i = token i), and the oracle encodes the same patterns in a process
pool.  Bar: bit-exact.
"""
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

CHUNK_LOG2 = 28
SUB_LOG2 = 24                     # patterns per worker task
N_KV, HD, BS = 8, 128, 16         # 1024 patterns per token, 16 tokens per block


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import paged_kv_cache_74_amd as pa
    pa.lib()
    return "cuda"


@pytest.fixture(scope="module")
def pool():
    # spawned workers (no copy of the GPU context); a worker that dies breaks the
    # pool with an error instead of being restarted
    n = min(16, len(os.sched_getaffinity(0)))
    with cf.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as p:
        yield p


@pytest.fixture(scope="module")
def buffers(dev):
    n = 1 << CHUNK_LOG2
    tokens = n // (N_KV * HD)
    blocks = tokens // BS
    src = torch.empty(n, dtype=torch.int32, device=dev)
    # the pool's torch dtype names the cache dtype: uint8 = FP8_E4M3, int8 = INT8
    kc = torch.empty((blocks, BS, N_KV, HD), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    slots = torch.arange(tokens, dtype=torch.int64, device=dev)
    return src, kc, vc, slots


@pytest.mark.parametrize("chunk", range(1 << (32 - CHUNK_LOG2)))
@pytest.mark.parametrize("codec", ["fp8", "int8"])
def test_every_fp32_pattern(dev, pool, buffers, codec, chunk):
    import paged_kv_cache_74_amd as pa
    from oracle_pool import encode_range
    src, kc, vc, slots = buffers
    n = 1 << CHUNK_LOG2
    start = chunk << CHUNK_LOG2
    print(f"{codec} patterns [{start:#x}, {start + n:#x})", flush=True)
    # the bit patterns start .. start + n - 1 (int64 -> int32 keeps the low 32 bits)
    src.copy_(torch.arange(start, start + n, dtype=torch.int64, device=dev).to(torch.int32))
    kc.fill_(0xAA)
    vc.fill_(0x55)
    rows = src.view(torch.float32).view(-1, N_KV, HD)
    if codec == "fp8":
        pa.pa_kv_append(kc, vc, rows, rows, slots, 1.0, 1.0)
    else:
        pa.pa_kv_append(kc.view(torch.int8), vc.view(torch.int8), rows, rows, slots, 1.0, 1.0)
    tasks = [(codec, start + (i << SUB_LOG2), 1 << SUB_LOG2) for i in range(n >> SUB_LOG2)]
    got_k = kc.view(-1).cpu().numpy()
    got_v = vc.view(-1).cpu().numpy()
    for i, ref in enumerate(pool.map(encode_range, tasks)):
        sl = slice(i << SUB_LOG2, (i + 1) << SUB_LOG2)
        for name, got in (("K", got_k[sl]), ("V", got_v[sl])):
            bad = np.flatnonzero(got != ref)
            assert bad.size == 0, (f"{codec} {name}: {bad.size} mismatches, first pattern "
                                   f"{start + (i << SUB_LOG2) + int(bad[0]):#010x}: gpu "
                                   f"{got[bad[0]]:#04x} oracle {ref[bad[0]]:#04x}")
