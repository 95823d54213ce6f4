"""LDS bank groups of the decode kernels' access patterns.

Runs pa_probe_lds_pattern once per pattern below (1024 one-wave workgroups,
1001 accesses each) and prints the patterns in launch order; run it under
rocprofv3 with the SQ_LDS_BANK_CONFLICT and SQ_ACTIVE_INST_LDS counters to
read the conflict cycles of each launch:

    rocprofv3 --pmc SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_WAVES \\
        --output-format csv -d OUT -- python3 -m paged_kv_cache_74_amd.probes.lds_banks

Lane l = 16 j + r.  The patterns are the decode kernels' (head_dim 128: V-slice
rows of 256 bytes, stage rows of 64 chunks of 16 bytes), each under the row
swizzle it has now (row_g), the one before it, and plain layouts.
"""
from __future__ import annotations


def row_g(t: int) -> int:
    return ((t & 7) << 1) | ((t >> 2) & 1)


def prev_g(t: int) -> int:     # the V-slice swizzle before row_g
    return ((t & 7) << 1) | ((t >> 3) & 1)


def _lanes():
    return [(l >> 4, l & 15) for l in range(64)]


def _tr(j, r):                 # transposed-read piece of lane (j, r): row, chunk of the pair, half
    return 4 * j + (r >> 2), (r >> 1) & 1, 8 * (r & 1)


def patterns():
    """(name, kind, 64 byte offsets)"""
    L = _lanes()
    return [
        ("write_b128 linear", "write_b128", [16 * l for l in range(64)]),
        ("write_b128 V slice, rows padded to 288 B", "write_b128", [r * 288 + 32 * j for j, r in L]),
        ("write_b128 V slice, previous swizzle", "write_b128", [r * 256 + 16 * ((2 * j) ^ prev_g(r)) for j, r in L]),
        ("write_b128 V slice, row_g", "write_b128", [r * 256 + 16 * ((2 * j) ^ row_g(r)) for j, r in L]),
        ("write_b128 V slice head_dim 64, t & 7", "write_b128", [r * 128 + 16 * ((2 * j) ^ (r & 7)) for j, r in L]),
        ("write_b128 stage, token row 1, row_g", "write_b128", [1024 + 16 * (l ^ row_g(1)) for l in range(64)]),
        ("read_b128 linear", "read_b128", [16 * l for l in range(64)]),
        ("read_b128 stage per-head, c ^ t", "read_b128", [r * 1024 + 16 * (j ^ r) for j, r in L]),
        ("read_b128 stage per-head, row_g", "read_b128", [r * 1024 + 16 * (j ^ row_g(r)) for j, r in L]),
        ("read_b64_tr_b16 linear", "read_b64_tr_b16", [8 * l for l in range(64)]),
        ("read_b64_tr_b16 V slice, rows padded to 288 B", "read_b64_tr_b16",
         [t * 288 + 16 * cb + h for t, cb, h in (_tr(j, r) for j, r in L)]),
        ("read_b64_tr_b16 V slice, previous swizzle", "read_b64_tr_b16",
         [t * 256 + 16 * (cb ^ prev_g(t)) + h for t, cb, h in (_tr(j, r) for j, r in L)]),
        ("read_b64_tr_b16 V slice, row_g", "read_b64_tr_b16",
         [t * 256 + 16 * (cb ^ row_g(t)) + h for t, cb, h in (_tr(j, r) for j, r in L)]),
        ("read_b64_tr_b16 V slice head_dim 64, t & 7", "read_b64_tr_b16",
         [t * 128 + 16 * (cb ^ (t & 7)) + h for t, cb, h in (_tr(j, r) for j, r in L)]),
        ("read_b64_tr_b16 bf16 stage, c ^ t", "read_b64_tr_b16",
         [t * 1024 + 16 * (cb ^ t) + h for t, cb, h in (_tr(j, r) for j, r in L)]),
        ("read_b64_tr_b16 bf16 stage, row_g", "read_b64_tr_b16",
         [t * 1024 + 16 * (cb ^ row_g(t)) + h for t, cb, h in (_tr(j, r) for j, r in L)]),
    ]


def main():
    import torch
    from . import pa_probe_lds_pattern
    wgs, iters = 1024, 1001
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    for i, (name, kind, offs) in enumerate(patterns()):
        assert all(0 <= o and o + 16 <= 16384 for o in offs), name
        pa_probe_lds_pattern(torch.tensor(offs, dtype=torch.int32, device="cuda"), kind, iters,
                             sink, wgs)
        torch.cuda.synchronize()
        print(f"launch {i}: {name}", flush=True)


if __name__ == "__main__":
    main()
