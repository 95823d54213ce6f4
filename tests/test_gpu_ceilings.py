"""The measured-ceiling probes read exactly the blocks they claim and issue the MFMAs they claim.

Each reader writes the XOR of every 32-bit word it read; the tests compare it
with NumPy's XOR of the same words (bit-exact).  The MFMA loop's sums are
exact in fp32 and compared with 64 * 16 * iters per wave.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from paged_kv_cache_74_amd import probes
    probes.lib()
    return "cuda"


def _xor(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel()))


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (10_000_048, 37), (64 << 20, 2048)])
def test_stream_read_reads_every_word_once(dev, nbytes, wgs):
    from paged_kv_cache_74_amd import probes
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.as_tensor(host.view(np.int32), device=dev)
    sink = torch.zeros(4 * wgs, dtype=torch.int32, device=dev)
    probes.pa_ceiling_stream_read(buf, sink, wgs)
    torch.cuda.synchronize()
    assert _xor(sink.cpu().numpy()) == _xor(host)


def test_gather_read_reads_the_listed_blocks(dev):
    from paged_kv_cache_74_amd import probes
    rng = np.random.default_rng(3)
    nb, bb = 50, 4096                                        # 50 blocks of 4 KiB
    k = rng.integers(0, 1 << 32, (nb, bb // 4), dtype=np.uint64).astype(np.uint32)
    v = rng.integers(0, 1 << 32, (nb, bb // 4), dtype=np.uint64).astype(np.uint32)
    blocks = rng.integers(0, nb, 301).astype(np.int32)
    blocks[[5, 77]] = [-3, nb + 9]                           # out of range: read block 0
    eff = np.where((blocks >= 0) & (blocks < nb), blocks, 0)
    want = 0
    for b in eff:
        want ^= _xor(k[b]) ^ _xor(v[b])
    gk = torch.as_tensor(k.view(np.int32), device=dev)
    gv = torch.as_tensor(v.view(np.int32), device=dev)
    sink = torch.zeros(4 * 64, dtype=torch.int32, device=dev)
    probes.pa_ceiling_gather_read(gk, gv, torch.as_tensor(blocks, device=dev), sink, 64)
    torch.cuda.synchronize()
    assert _xor(sink.cpu().numpy()) == want


def test_mfma_loop_sums(dev):
    from paged_kv_cache_74_amd import probes
    W, iters = 16, 300
    sink = torch.zeros(4 * W, dtype=torch.float32, device=dev)
    probes.pa_ceiling_mfma_bf16(sink, W, iters)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 64.0 * 16 * iters).all()


def test_mfma_lds_operand_loop_sums(dev):
    """The loop with its A operands read from LDS (bf16 1.0) sums as the register loop."""
    from paged_kv_cache_74_amd import probes
    W, iters = 16, 300
    sink = torch.zeros(4 * W, dtype=torch.float32, device=dev)
    probes.pa_ceiling_mfma_bf16_lds(sink, W, iters)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 64.0 * 16 * iters).all()


def _lds_elements_xor(offsets, nbytes):
    """XOR of the 16-bit elements a wave reads: each lane's nbytes at its offset, the LDS
    area holding element k = (k * 40503) mod 2^16."""
    x = 0
    for o in offsets:
        for k in range(o // 2, (o + nbytes) // 2):
            x ^= (k * 40503) & 0xFFFF
    return x


def test_lds_pattern_probe_reads_what_each_lane_addresses(dev):
    """Every read pattern of the bank-group probe (odd repeat count) returns the XOR of the
    elements at the lanes' offsets; writes return 0.  The transposed read spreads the same
    elements over other lanes, so its wave XOR is the same."""
    from paged_kv_cache_74_amd import probes
    from paged_kv_cache_74_amd.probes import lds_banks
    size = {"read_b128": 16, "read_b64_tr_b16": 8, "read_b64": 8}
    W = 4
    sink = torch.zeros(W, dtype=torch.int32, device=dev)
    for name, kind, offs in lds_banks.patterns() + [("b64 linear", "read_b64", [8 * l for l in range(64)])]:
        probes.pa_probe_lds_pattern(torch.tensor(offs, dtype=torch.int32, device=dev), kind, 3,
                                    sink, W)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        want = 0 if kind == "write_b128" else _lds_elements_xor(offs, size[kind])
        assert (got == want).all(), (name, got, want)
