#!/usr/bin/env python3
"""Benchmark of the paged-KV decode step on one MI355X.

One step = the whole hot path over one batch: slot mapping of the step's new
tokens and KV append (scatter into the paged pool), then paged decode attention
(split kernel + log-sum-exp merge).  A decode step whose one new token per
sequence is the last of its context appends inside the split kernel
(pa_decode_append_partials); otherwise the append runs first, in one launch
(pa_kv_append_paged) when the step's segments are short, else as two calls
(--separate-append / --two-call-append force those forms).  Default workload: Llama-3-8B-shaped GQA
decode -- batch 64, 32 query / 8 KV heads, head_dim 128, block 16, bf16,
context lengths ~ U{2048..8192}, 19 sequences sharing an 800-token prefix
through shared physical blocks, one appended token per sequence.

Inputs are resident in HBM before timing.  Several copies of the pool are
rotated so a step never finds the previous step's K/V in L2 or the MALL.
Prints ONE JSON line on stdout (human-readable detail goes to stderr).

    python bench.py [--steps K] [--warmup W] [--workload llama3-gqa|llama2|longtail|longtail-fp8|...]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "decode paged-attn achieved HBM GB/s (% of peak) + seqs·tokens/s, 1×MI355X"

WORKLOADS = {
    "llama3-gqa": (3, "bf16"),
    "llama2": (2, "bf16"),
    "longtail": (4, "bf16"),
    "longtail-fp8": (4, "fp8"),
    "longtail-int8": (4, "int8"),
    "longtail-int4": (4, "int4"),
    "mixed": (5, "bf16"),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(w, seqs=None):
    """4 * head_dim * n_q_heads flops per visible (query, key) pair (QK^T and PV)."""
    pairs = 0
    for s in range(w.num_prefill_seqs) if seqs is None else seqs:
        L, T = int(w.q_lens[s]), int(w.context_lens[s])
        pairs += L * (T - L) + L * (L + 1) // 2 if w.causal else L * T
    return 4.0 * w.head_dim * w.n_q_heads * pairs


def byte_model(w):
    """Algorithmic bytes of one step (what the method must move)."""
    eb = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1, "int4": 0.5}[w.cache_dtype]
    qb = {"f32": 4, "bf16": 2}[w.q_dtype]
    sb = {"f32": 4, "bf16": 2}[w.src_dtype]
    nkv, hd, bs = w.n_kv_heads, w.head_dim, w.block_size
    # int4: each (token, head) also carries its float32 value scale
    tok_head = hd * 2 * eb + (4 if w.cache_dtype == "int4" else 0)
    rows = list(w.decode_rows)
    ctx = w.context_lens[rows].astype(float)
    kv_logical = float(ctx.sum()) * nkv * tok_head
    shared = max(len(w.shared_prefix_seqs) - 1, 0) * w.shared_prefix_blocks * bs
    kv_unique = kv_logical - shared * nkv * tok_head
    B = len(rows)
    q_bytes = B * w.n_q_heads * hd * qb
    table_bytes = float(sum(math.ceil(c / bs) for c in ctx)) * 4 + B * 4
    chan_bytes = nkv * hd * 4 if w.cache_dtype == "int4" else 0   # int4 key scales
    split = kv_unique + q_bytes + table_bytes + chan_bytes
    out_bytes = B * w.n_q_heads * hd * qb
    n_new = int(w.new_len.sum())
    append = n_new * nkv * (hd * (sb + eb) * 2 + (4 if w.cache_dtype == "int4" else 0)) + n_new * 8
    slots = n_new * (8 + 4) + B * 8
    return {"kv_logical": kv_logical, "kv_unique": kv_unique, "split_kernel": split,
            "step": split + out_bytes + append + slots, "append": append,
            # the split kernel that also appends the step's tokens (pa_decode_append)
            "split_append_kernel": split + append}


DECODE_SOURCES = ("paged_kv_cache_74_amd/csrc/decode.hip", "paged_kv_cache_74_amd/csrc/pa_device.h",
                  "paged_kv_cache_74_amd/csrc/internal.h")
PREFILL_SOURCES = ("paged_kv_cache_74_amd/csrc/prefill.hip", "paged_kv_cache_74_amd/csrc/pa_device.h",
                   "paged_kv_cache_74_amd/csrc/internal.h")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def source_hash(sources) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def timed(fn, reps: int = 3, burst: int = 8) -> float:
    """Milliseconds per launch of fn(): the median over reps of a burst of back-to-back
    launches between two HIP events on the current stream, divided by the burst (so the
    host's launch overhead overlaps the GPU's work instead of being timed), after one
    warm-up."""
    import numpy as np
    import torch
    fn()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(burst):
            fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / burst)
    return float(np.median(ts))


def measure_ceilings(w, dw, kc, vc, dev, want_mfma: bool):
    """What plain readers and a plain MFMA loop reach on this GPU (see pa.h, Measured
    ceilings): the decode rows' whole K and V blocks read in table order (the pattern a
    paged decode reads), the whole pools read in physical order, and the bf16 MFMA
    issue rate."""
    import numpy as np
    import torch

    from paged_kv_cache_74_amd import probes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 16 * 4, dtype=torch.int32, device=dev)
    rec = {}
    block_bytes = kc.numel() * kc.element_size() // kc.shape[0]
    rows = list(w.decode_rows)
    nblk = [-(-int(w.context_lens[s]) // w.block_size) for s in rows]
    blocks = np.concatenate([w.block_tables[s, :n] for s, n in zip(rows, nblk)]).astype(np.int32)
    for name, lst in (("table_order", blocks), ("physical_order", np.arange(kc.shape[0]))):
        gb = torch.as_tensor(lst.astype(np.int32), device=dev)
        # the best of 4, 8 and 16 workgroups per CU
        ms = min(timed(lambda: probes.pa_ceiling_gather_read(kc, vc, gb, sink, W))
                 for W in (cus * 4, cus * 8, cus * 16))
        rec[f"block_read_{name}_GBps"] = round(2 * lst.size * block_bytes / (ms * 1e-3) / 1e9, 1)
    rec["block_read_table_order_bytes"] = int(2 * blocks.size * block_bytes)
    nbytes = kc.numel() * kc.element_size()
    ms = min(timed(lambda: probes.pa_ceiling_stream_read(kc, sink, W))
             for W in (cus * 4, cus * 8, cus * 16))
    rec["contiguous_read_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    if want_mfma:
        Wm, iters = cus * 2, 4000
        fsink = torch.empty(4 * Wm, dtype=torch.float32, device=dev)
        ms = timed(lambda: probes.pa_ceiling_mfma_bf16(fsink, Wm, iters))
        rec["mfma_bf16_TFLOPs"] = round(Wm * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12, 1)
        # with one operand from LDS per MFMA, as prefill reads K and V^T: the best
        # of two and three workgroups per CU (prefill runs three)
        best = 0.0
        for Wl in (cus * 2, cus * 3):
            fs = torch.empty(4 * Wl, dtype=torch.float32, device=dev)
            ms = timed(lambda: probes.pa_ceiling_mfma_bf16_lds(fs, Wl, iters))
            best = max(best, Wl * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12)
        rec["mfma_bf16_lds_operand_TFLOPs"] = round(best, 1)
    return rec


def decode_kernel(w) -> str:
    """The split kernel pa_decode_partials launches for this workload's cache."""
    if w.block_size >= 16 and w.cache_dtype in ("bf16", "fp8", "int8", "int4"):
        return "decode_mfma_kernel"
    return "decode_split_kernel"


def measured_traffic(workload: str, kernel: str, sources):
    """HBM bytes per launch of `kernel` from the committed counter record, or
    None when there is no record for this workload or the kernel sources changed."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(f"{workload}:{kernel}")
    if not r or r.get("source_sha256") != source_hash(sources):
        return None
    return r["fetch_kib"] * r["fetch_scale"] * 1024 + r["write_kib"] * r["write_scale"] * 1024


def _oracle_worker(job):
    """One host core's share of the oracle baseline (runs in a spawned process with one
    BLAS thread): for each task, build the oracle pools it reads (setup, not timed),
    then time the oracle on it, until the timed total reaches the budget.

    Tasks: ("decode", s) -- slot map + append of sequence s's new token + decode of s;
    ("prefill", s, i) -- chunk s's query row i as a chunk of its own (its causal
    context).  Returns {kind: [seconds, bytes, flops, count]}."""
    import numpy as np

    import oracle
    w, files, tasks, budget_s = job
    a = {k: np.load(f, mmap_mode="r") for k, f in files.items()}
    paged = oracle.paged
    src, cdt, bs = w.src_dtype, w.cache_dtype, w.block_size
    int4 = cdt == "int4"
    hd_store = w.head_dim // 2 if int4 else w.head_dim
    dt = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8, "int8": np.uint8,
          "int4": np.uint8}[cdt]
    shape = (w.num_blocks, bs, w.n_kv_heads, hd_store)
    pk, pv = np.zeros(shape, dt), np.zeros(shape, dt)          # pages touched on demand
    ps = np.zeros((w.num_blocks, w.n_kv_heads, bs), np.float32) if int4 else None
    res_cu, new_cu, q_cu = w.cu(w.res_len), w.cu(w.new_len), w.cu(w.q_lens)
    eb = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1, "int4": 0.5}[cdt]
    tok_head = w.head_dim * 2 * eb + (4 if int4 else 0)

    def append(r, which):
        start, lens, kk, vv, cu = ((w.res_start, w.res_len, a["res_k"], a["res_v"], res_cu)
                                   if which == "res" else
                                   (w.new_start, w.new_len, a["new_k"], a["new_v"], new_cu))
        sl = paged.slot_mapping(w.block_tables[[r]], start[[r]], lens[[r]], bs)
        k, v = np.asarray(kk[cu[r]:cu[r + 1]]), np.asarray(vv[cu[r]:cu[r + 1]])
        if int4:
            paged.kv_append_int4(pk, pv, ps, k, v, sl, bs, src, w.k_channel_scales)
        else:
            paged.kv_append(pk, k, sl, bs, src, cdt, w.k_scale)
            paged.kv_append(pv, v, sl, bs, src, cdt, w.v_scale)

    ready = set()
    out = {}
    t_total, done = 0.0, 0
    while True:
        for task in tasks:
            if done and t_total >= budget_s:
                return out
            kind, s = task[0], task[1]
            seqs = [s]
            if w.shared_prefix_seqs and s in w.shared_prefix_seqs[1:]:
                seqs = [w.shared_prefix_seqs[0], s]
            for r in seqs:                              # resident tokens: setup, not timed
                if r not in ready:
                    ready.add(r)
                    append(r, "res")
                    if kind == "prefill":
                        append(r, "new")                # the chunk's own K/V
            if kind == "decode":
                qd = np.zeros((w.num_seqs,) + a["q"].shape[1:], a["q"].dtype)
                qd[s] = a["q"][q_cu[s]]
                t0 = time.perf_counter()                # timed: slot map + append + decode
                append(s, "new")
                if int4:
                    paged.decode_int4(qd, w.q_dtype, pk, pv, ps, w.k_channel_scales,
                                      w.block_tables, w.context_lens, bs, w.group_size,
                                      w.scale, rows=[s])
                else:
                    paged.decode(qd, w.q_dtype, pk, pv, cdt, w.block_tables, w.context_lens, bs,
                                 w.group_size, w.scale, w.k_scale, w.v_scale, rows=[s])
                dt_s = time.perf_counter() - t0
                nbytes, nflops = float(w.context_lens[s]) * w.n_kv_heads * tok_head, 0.0
            else:
                i = task[2]
                row = int(q_cu[s]) + i
                T = int(w.context_lens[s]) - int(w.q_lens[s]) + i + 1
                t0 = time.perf_counter()                # timed: one query row of the chunk
                paged.prefill_chunk(np.asarray(a["q"][row:row + 1]), w.q_dtype, np.array([0, 1]),
                                    pk, pv, cdt, w.block_tables[s:s + 1], np.array([T]), bs,
                                    w.group_size, w.scale, True, w.k_scale, w.v_scale)
                dt_s = time.perf_counter() - t0
                nbytes, nflops = 0.0, 4.0 * w.head_dim * w.n_q_heads * T
            acc = out.setdefault(kind, [0.0, 0.0, 0.0, 0])
            acc[0] += dt_s
            acc[1] += nbytes
            acc[2] += nflops
            acc[3] += 1
            t_total += dt_s
            done += 1


def cpu_baseline(w, budget_s: float, step_bytes: float, step_flops: float):
    """The oracle, as it is, on a bounded sample of the same step, on the host cores:
    one spawned worker process per core (up to 16), each with one BLAS thread (a
    per-(sequence, head) product does not spread over BLAS threads), each timing its
    share for about budget_s seconds.  Scaled to the step: the oracle's time for the
    whole step on these cores is step_bytes at the decode rate plus step_flops at the
    prefill rate; value = step_bytes / that time (the unit of the step's value)."""
    import concurrent.futures as cf
    import dataclasses
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np

    from workloads import codes

    n = max(1, min(16, len(os.sched_getaffinity(0))))
    tmp = tempfile.mkdtemp(prefix="pa_oracle_")
    try:
        files = {}
        for name, dtype in (("q", w.q_dtype), ("res_k", w.src_dtype), ("res_v", w.src_dtype),
                            ("new_k", w.src_dtype), ("new_v", w.src_dtype)):
            files[name] = os.path.join(tmp, name + ".npy")
            np.save(files[name], codes(getattr(w, name), dtype))
        meta = dataclasses.replace(w, q=None, res_k=None, res_v=None, new_k=None, new_v=None)
        tasks = [("decode", s) for s in w.decode_rows]
        rng = np.random.default_rng(0)
        for s in range(w.num_prefill_seqs):             # sampled query rows of each chunk
            L = int(w.q_lens[s])
            for i in sorted(set([0, L - 1] + rng.integers(0, L, 6).tolist())):
                tasks.append(("prefill", s, i))
        order = rng.permutation(len(tasks))
        shares = [[tasks[k] for k in order[j::n]] for j in range(n)]
        shares = [sh for sh in shares if sh]
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                              "MKL_NUM_THREADS")}
        os.environ.update({k: "1" for k in env})        # inherited by the spawned workers
        try:
            t0 = time.perf_counter()
            with cf.ProcessPoolExecutor(len(shares), mp_context=mp.get_context("spawn")) as ex:
                res = list(ex.map(_oracle_worker, [(meta, files, sh, budget_s) for sh in shares]))
            wall = time.perf_counter() - t0
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    cores = len(shares)
    tot = {}
    for r in res:
        for kind, acc in r.items():
            t = tot.setdefault(kind, [0.0, 0.0, 0.0, 0])
            for k in range(4):
                t[k] += acc[k]
    # per core-second rates, times the cores that ran them side by side
    t_step = 0.0
    sample = []
    if "decode" in tot:
        sec, by, _, cnt = tot["decode"]
        gbs = cores * by / sec / 1e9
        t_step += step_bytes / (gbs * 1e9)
        sample.append(f"{cnt} sequence decodes (slot map + append + decode of one sequence, "
                      f"{sec:.1f} core-s, {gbs:.3f} GB/s of logical K/V on {cores} cores)")
    if "prefill" in tot:
        sec, _, fl, cnt = tot["prefill"]
        gfs = cores * fl / sec / 1e9
        t_step += step_flops / (gfs * 1e9)
        sample.append(f"{cnt} chunk query rows ({sec:.1f} core-s, {gfs:.3f} GFLOP/s of visible "
                      f"pairs on {cores} cores)")
    rec = {"value": round(step_bytes / t_step / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": "; ".join(sample) + f"; {wall:.1f} s wall, one process per core, float64 "
                     f"NumPy; scaled to the step ({step_bytes / 1e9:.3f} GB"
                     + (f" + {step_flops / 1e9:.1f} GFLOP" if step_flops else "") + ")",
           "oracle_step_ms": round(t_step * 1e3, 3)}
    if "decode" in tot:
        rec["decode_GBps"] = round(gbs, 4)
    if "prefill" in tot:
        rec["prefill_GFLOPs"] = round(gfs, 4)
    return rec


# Block copies on the Llama-3-8B-shaped pool (block 16, 8 KV heads, 128 dims, bf16:
# 32 KiB of K and 32 KiB of V per block): copy-on-write of 4096 blocks within the
# device pool, and a swap of 4096 blocks out to pinned host memory and back in.
BLOCK_WORKLOADS = {"cow": 4096, "swap": 4096}
HOST_LINK_PEAK_GBS = 64.0      # PCIe 5.0 x16, one direction


def block_copy_bench(args, torch, np, pa):
    """K copy calls of n block pairs; algorithmic bytes = pairs * 2 (K, V) * block bytes
    * 2 (read + write)."""
    dev = "cuda"
    nb, bs, nkv, hd = 19850, 16, 8, 128
    n = BLOCK_WORKLOADS[args.workload]
    block_bytes = bs * nkv * hd * 2
    gen = torch.Generator(device=dev).manual_seed(0)
    k = torch.empty((nb, bs, nkv, hd), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    k.view(torch.int16).random_(generator=gen)
    v.view(torch.int16).random_(generator=gen)
    perm = np.random.default_rng(0).permutation(nb)
    if args.workload == "cow":
        pairs = torch.as_tensor(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64), device=dev)
        calls = [lambda: pa.pa_copy_blocks(k, v, k, v, pairs)]
        bound, peak = "hbm", HBM_PEAK_GBS
        what = f"copy-on-write of {n} blocks within the device pool"
    else:
        hk = torch.empty((n, bs, nkv, hd), dtype=torch.bfloat16, pin_memory=True)
        hv = torch.empty_like(hk, pin_memory=True)
        out_pairs = torch.as_tensor(np.stack([perm[:n], np.arange(n)], 1).astype(np.int64), device=dev)
        in_pairs = torch.as_tensor(np.stack([np.arange(n), perm[n:2 * n]], 1).astype(np.int64),
                                   device=dev)
        calls = [lambda: pa.pa_copy_blocks(hk, hv, k, v, out_pairs),
                 lambda: pa.pa_copy_blocks(k, v, hk, hv, in_pairs)]
        bound, peak = "host-link", HOST_LINK_PEAK_GBS
        what = f"swap of {n} blocks out to pinned host memory and back in"
    nbytes = n * 2 * block_bytes            # bytes copied per call (K and V)
    # bytes the bound resource carries per call: HBM reads and writes them (copy-on-write);
    # the host link carries them once (swap)
    moved = 2 * nbytes if bound == "hbm" else nbytes
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps * len(calls))]
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for j, c in enumerate(calls):
            e = ev[i * len(calls) + j]
            e[0].record(stream)
            c()
            e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    per_call = float(ms.mean())
    gbs = moved / (per_call * 1e-3) / 1e9
    step_ms = wall * 1e3 / args.steps
    log(f"{what}: {per_call * 1e3:.1f} us per call -> {gbs:.1f} GB/s through the {bound} "
        f"({gbs / peak:.1%} of {peak:.0f} GB/s)")
    # measured ceiling: the same bytes as one contiguous copy (device to device, or out to
    # pinned host memory and back) through torch's copy, timed the same way
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if bound == "hbm":
        dst = torch.empty_like(src)
        ops = [lambda: dst.copy_(src)]
    else:
        host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        ops = [lambda: host.copy_(src, non_blocking=True), lambda: src.copy_(host, non_blocking=True)]
    for _ in range(args.warmup):
        for o in ops:
            o()
    torch.cuda.synchronize()
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps * len(ops))]
    for i in range(args.steps):
        for j, o in enumerate(ops):
            e = cev[i * len(ops) + j]
            e[0].record(stream)
            o()
            e[1].record(stream)
    torch.cuda.synchronize()
    ceil_gbs = moved / (float(np.mean([a.elapsed_time(b) for a, b in cev])) * 1e-3) / 1e9
    log(f"contiguous copy of the same bytes: {ceil_gbs:.1f} GB/s -> the block copy at "
        f"{gbs / ceil_gbs:.1%} of it")
    rec = {"metric": f"block copy GB/s ({args.workload})", "value": round(moved * len(calls) /
           (step_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": what, "blocks": n, "block_bytes_k": block_bytes,
                      "pool_blocks": nb},
           "roofline": {"kernel": "copy_blocks_kernel (pa_copy_blocks)", "bound": bound,
                        "achieved": round(gbs, 2), "peak": peak, "unit": "GB/s",
                        "frac": round(gbs / peak, 4), "traffic": None,
                        "avg_launch_us": round(per_call * 1e3, 2),
                        "algorithmic_bytes_per_launch": moved},
           "cpu_baseline": None,
           "measured_ceiling": {"what": "contiguous copy of the same bytes (torch copy_)",
                                "gbs": round(ceil_gbs, 2), "frac": round(gbs / ceil_gbs, 4)}}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3-gqa",
                    choices=sorted(WORKLOADS) + sorted(BLOCK_WORKLOADS))
    ap.add_argument("--pools", type=int, default=2, help="pool copies rotated across steps")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="timed oracle seconds per host core for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured-ceiling probes (contiguous read, block-order read, "
                         "MFMA loop)")
    ap.add_argument("--two-call-append", action="store_true",
                    help="append through pa_slot_mapping + pa_kv_append[_int4] instead of the "
                         "one-launch pa_kv_append[_int4]_paged")
    ap.add_argument("--separate-append", action="store_true",
                    help="decode workloads: append in its own launch (pa_kv_append_paged) before "
                         "pa_decode_partials, instead of pa_decode_append_partials")
    ap.add_argument("--one-launch", action="store_true",
                    help="mixed workload: chunks and decode rows in one pa_prefill_chunk call "
                         "(its query-length-1 rows take the decode kernel's path inside the call)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this size (for scaling HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_74_amd as pa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        # a copy kernel of known size: FETCH_SIZE / WRITE_SIZE per dispatch should
        # read copy_calibration_mib MiB each; their ratio scales the counters
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration_mib} MiB x 3")
        return
    if args.workload in BLOCK_WORKLOADS:
        return block_copy_bench(args, torch, np, pa)
    cfg, kv = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    w = workloads.full(cfg, kv=kv)
    workloads.draw_values(w, dev)
    from workloads.device import DeviceWorkload, i32
    dw = DeviceWorkload(w, dev)
    dw.append_resident()
    int4 = w.cache_dtype == "int4"
    if int4 and args.one_launch:
        log("--one-launch takes the per-tensor-scale caches only")
        sys.exit(2)
    pools = [(dw.k_cache, dw.v_cache, dw.v_scales if int4 else None)]
    for _ in range(max(args.pools, 1) - 1):
        pools.append((dw.k_cache.clone(), dw.v_cache.clone(),
                      dw.v_scales.clone() if int4 else None))
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t0:.1f} s: {w.name}, {w.num_seqs} seqs, "
        f"{w.num_blocks} blocks, pool {2 * dw.k_cache.numel() * dw.k_cache.element_size() / 2**30:.2f} GiB x {len(pools)}")

    # step inputs, resident in HBM
    q, tables, ctx = dw.decode_inputs()
    B = q.shape[0]
    maxc = int(w.context_lens[list(w.decode_rows)].max())
    new_cu = i32(w.cu(w.new_len), dev)
    new_start = i32(w.new_start, dev)
    n_new = int(w.new_len.sum())
    new_k, new_v = w.new_k.to(dev), w.new_v.to(dev)
    slots = torch.empty(n_new, dtype=torch.int64, device=dev)
    out = torch.empty_like(q)
    ws = pa.workspace(pa.pa_decode_workspace_bytes(B, w.n_q_heads, w.n_kv_heads, w.head_dim, maxc,
                                                   args.split_tokens), dev)
    stream = torch.cuda.current_stream()

    P = w.num_prefill_seqs
    one = args.one_launch
    if one and not P:
        log("--one-launch needs a workload with prefill chunks (mixed)")
        sys.exit(2)
    if P:
        # one call: the whole batch (chunks, then the decode rows as chunks of
        # one query); else the chunks only, the decode rows going to pa_decode
        PB = w.num_seqs if one else P
        pf_cu = i32(w.cu(w.q_lens[:PB]), dev)
        pf_q = dw.q[: int(w.q_lens[:PB].sum())]
        pf_out = torch.empty_like(pf_q)
        pf_maxq, pf_maxc = int(w.q_lens[:PB].max()), int(w.context_lens[:PB].max())
        pf_ws = pa.workspace(pa.pa_prefill_workspace_bytes(
            PB, pf_q.shape[0], pf_maxq, w.n_q_heads, w.n_kv_heads, w.head_dim, pf_maxc), dev)

    max_new = int(w.new_len.max())
    # The one-launch append sizes its grid by the longest segment; with a few
    # long chunks among many one-token rows (the mixed step) most of that grid
    # is idle, and the two calls are faster (915 against 920 us per step).
    two_calls = args.two_call_append or max_new * len(w.new_len) > 4 * n_new
    # a decode step whose new token per sequence is the last of its context: the
    # split kernel appends it (pa_decode_append_partials), one launch fewer
    fused = (not P and not int4 and not args.separate_append and not args.two_call_append
             and bool((w.new_len == 1).all()) and bool((w.new_start == w.context_lens - 1).all()))

    def step(i, ev=None, pev=None):
        kc, vc, vsc = pools[i % len(pools)]
        if fused:
            if ev is not None:
                ev[0].record(stream)
            pa.pa_decode_append_partials(q, kc, vc, new_k, new_v, tables, ctx, maxc, w.scale, ws,
                                         w.k_scale, w.v_scale, args.split_tokens,
                                         slot_mapping=slots)
            if ev is not None:
                ev[1].record(stream)
            pa.pa_decode_merge(out, ctx, w.n_kv_heads, maxc, ws,
                               w.v_scale if w.cache_dtype in ("fp8", "int8") else 1.0,
                               args.split_tokens)
            return
        if two_calls:
            pa.pa_slot_mapping(dw.tables, new_cu, new_start, w.block_size, n_new, out=slots)
            if int4:
                pa.pa_kv_append_int4(kc, vc, vsc, new_k, new_v, slots, dw.k_channel_scales)
            else:
                pa.pa_kv_append(kc, vc, new_k, new_v, slots, w.k_scale, w.v_scale)
        elif int4:
            pa.pa_kv_append_int4_paged(kc, vc, vsc, new_k, new_v, dw.tables, new_cu, new_start,
                                       max_new, dw.k_channel_scales, slot_mapping=slots)
        else:
            pa.pa_kv_append_paged(kc, vc, new_k, new_v, dw.tables, new_cu, new_start, max_new,
                                  slot_mapping=slots, k_scale=w.k_scale, v_scale=w.v_scale)
        if P:
            if pev is not None:
                pev[0].record(stream)
            pa.pa_prefill_chunk(pf_q, kc, vc, pf_cu, dw.tables[:PB], dw.ctx[:PB], pf_maxq, pf_maxc,
                                w.scale, causal=True, k_scale=w.k_scale, v_scale=w.v_scale,
                                out=pf_out, ws=pf_ws)
            if pev is not None:
                pev[1].record(stream)
        if one:
            return
        if ev is not None:
            ev[0].record(stream)
        if int4:
            pa.pa_decode_int4_partials(q, kc, vc, vsc, dw.k_channel_scales, tables, ctx, maxc,
                                       w.scale, ws, args.split_tokens)
        else:
            pa.pa_decode_partials(q, kc, vc, tables, ctx, maxc, w.scale, ws, w.k_scale,
                                  args.split_tokens)
        if ev is not None:
            ev[1].record(stream)
        pa.pa_decode_merge(out, ctx, w.n_kv_heads, maxc, ws, w.v_scale if w.cache_dtype in ("fp8", "int8") else 1.0,
                           args.split_tokens)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1: K steps back to back (no events inside) -> value, ms_per_step
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # timed region 2: the same K steps with HIP events (on the launch stream)
    # around the split kernel -> its average launch duration (roofline)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    pevents = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events[i], pevents[i])
    torch.cuda.synchronize()
    split_ms = np.array([a.elapsed_time(b) for a, b in events]) if not one else None
    prefill_ms = np.array([a.elapsed_time(b) for a, b in pevents]) if P else None

    bm = byte_model(w)
    ms_step = wall * 1e3 / args.steps
    step_gbs = bm["step"] / (ms_step * 1e-3) / 1e9
    ctx_tokens = float(w.context_lens[list(w.decode_rows)].sum())
    split_bytes = bm["split_append_kernel"] if fused else bm["split_kernel"]
    if not one:
        split_avg = float(split_ms.mean())
        achieved = split_bytes / (split_avg * 1e-3) / 1e9
        log(f"step {ms_step * 1e3:.1f} us ({step_gbs:.0f} GB/s); split kernel avg {split_avg * 1e3:.1f} us "
            f"(p10 {np.percentile(split_ms, 10) * 1e3:.1f}, p90 {np.percentile(split_ms, 90) * 1e3:.1f}) "
            f"-> {achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.1%} of 8 TB/s; "
            f"KV unique {bm['kv_unique'] / 1e9:.3f} GB, logical {bm['kv_logical'] / 1e9:.3f} GB")

    prefill_rec = None
    if P:
        fl = prefill_flops(w, range(PB))
        pf_avg = float(prefill_ms.mean())
        tf = fl / (pf_avg * 1e-3) / 1e12
        what = ("pa_prefill_chunk: chunks and decode rows in one call" if one
                else "pa_prefill_chunk")
        prefill_rec = {"kernel": f"prefill_kernel ({what})", "bound": "mfma",
                       "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                       "traffic": measured_traffic(args.workload + ("-one" if one else ""),
                                                   "prefill_kernel", PREFILL_SOURCES),
                       "avg_launch_us": round(pf_avg * 1e3, 2),
                       "launch_us_p10_p50_p90": [round(float(np.percentile(prefill_ms, q)) * 1e3, 2)
                                                 for q in (10, 50, 90)],
                       "flops_per_launch": fl}
        log(f"prefill avg {pf_avg * 1e3:.1f} us -> {tf:.1f} TFLOP/s = {tf / MFMA_BF16_PEAK_TFLOPS:.1%} "
            f"of the bf16 MFMA peak ({fl / 1e9:.1f} GFLOP)")
        if one:
            # lower bound of the one call: the chunks' flops at the MFMA peak
            # plus the decode rows' bytes at the HBM peak
            t_min = (prefill_flops(w) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                     + bm["split_kernel"] / (HBM_PEAK_GBS * 1e9))
            prefill_rec["serial_bound_us"] = round(t_min * 1e6, 2)
            prefill_rec["frac_of_serial_bound"] = round(t_min / (pf_avg * 1e-3), 4)
            log(f"step {ms_step * 1e3:.1f} us ({step_gbs:.0f} GB/s), one call; bound "
                f"{t_min * 1e6:.1f} us (chunk flops at the MFMA peak + decode bytes at the HBM peak) "
                f"= {t_min / (pf_avg * 1e-3):.1%} of the call")

    ceil = None
    if not args.no_ceilings:
        kc0, vc0, _ = pools[0]
        ceil = measure_ceilings(w, dw, kc0, vc0, dev, want_mfma=bool(P))
        tbl = ceil["block_read_table_order_GBps"]
        msg = (f"measured ceilings: the decode rows' blocks read in table order {tbl:.0f} GB/s, "
               f"the pools in physical order {ceil['block_read_physical_order_GBps']:.0f} GB/s, "
               f"the K pool as one contiguous read {ceil['contiguous_read_GBps']:.0f} GB/s")
        if not one:
            logical = bm["kv_logical"] / (split_avg * 1e-3) / 1e9
            ceil["split_kernel_logical_GBps"] = round(logical, 1)
            ceil["split_kernel_frac_of_table_order_read"] = round(logical / tbl, 4)
            msg += f" (split kernel: {logical:.0f} GB/s of logical K/V = {logical / tbl:.1%} of the first)"
        if "mfma_bf16_TFLOPs" in ceil:
            msg += (f", bf16 MFMA loop {ceil['mfma_bf16_TFLOPs']:.0f} TFLOP/s "
                    f"({ceil['mfma_bf16_lds_operand_TFLOPs']:.0f} with one operand from LDS)")
            if prefill_rec:
                prefill_rec["frac_of_mfma_loop"] = round(
                    prefill_rec["achieved"] / ceil["mfma_bf16_TFLOPs"], 4)
                prefill_rec["frac_of_lds_operand_loop"] = round(
                    prefill_rec["achieved"] / ceil["mfma_bf16_lds_operand_TFLOPs"], 4)
        log(msg)

    cpu = None
    if not args.no_cpu_baseline:
        for name in ("q", "res_k", "res_v", "new_k", "new_v"):
            setattr(w, name, getattr(w, name).cpu())
        cpu = cpu_baseline(w, args.cpu_seconds, bm["step"],
                           prefill_flops(w, range(P)) if P else 0.0)
        log(f"cpu baseline (oracle): {cpu['value']} GB/s, {cpu['sample']}")

    rec = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.cache_dtype == "bf16" else f"bf16-q/{w.cache_dtype}-kv",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: " + ("paged step, one attention launch (slot map + KV append + "
                                         "chunks and decode rows in pa_prefill_chunk)" if one else
                                         "paged decode step (slot map + KV append + split-K decode + merge)"),
            "append": "in the split kernel (pa_decode_append_partials)" if fused else
                      "pa_slot_mapping + pa_kv_append" if two_calls else
                      "pa_kv_append_paged (slot map and append in one launch)",
            "batch": B, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": w.cache_dtype,
            "context_tokens": int(ctx_tokens), "max_context": maxc,
            "shared_prefix_seqs": len(w.shared_prefix_seqs),
            "shared_prefix_tokens": w.shared_prefix_blocks * w.block_size,
            "appended_tokens": n_new, "pool_copies_rotated": len(pools),
            "split_tokens": args.split_tokens or "auto",
        },
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(B / (ms_step * 1e-3), 1),
        "context_tokens_per_s": round(ctx_tokens / (ms_step * 1e-3), 1),
        "bytes_per_step": {"algorithmic_unique": bm["step"], "kv_unique": bm["kv_unique"],
                           "kv_logical": bm["kv_logical"]},
        "roofline": prefill_rec if one else {
            "kernel": f"{decode_kernel(w)} (" + ("pa_decode_append_partials: append + split"
                                                 if fused else "pa_decode_partials") + ")",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload, decode_kernel(w), DECODE_SOURCES),
            "avg_launch_us": round(split_avg * 1e3, 2),
            "launch_us_p10_p50_p90": [round(float(np.percentile(split_ms, q)) * 1e3, 2)
                                      for q in (10, 50, 90)],
            "algorithmic_bytes_per_launch": split_bytes,
        },
        "cpu_baseline": cpu,
        "measured_ceilings": ceil,
    }
    if prefill_rec and not one:
        rec["prefill_roofline"] = prefill_rec
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
