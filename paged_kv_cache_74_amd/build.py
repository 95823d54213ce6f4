"""Build the HIP libraries in-tree for gfx950.

    python -m paged_kv_cache_74_amd.build        # or __graft_entry__.build()

libpa.so, the paged-KV attention library (C ABI in include/pa.h), is linked
from csrc/*.hip.  libpa_probes.so, the benchmark's measurement probes
(probes/pa_probes.h), is linked from probes/*.hip on its own, so the product
library exports only the method's entry points.  Every source is compiled to
an object with hipcc each time build() is called.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
PROBES = os.path.join(HERE, "probes")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa.so")
PROBES_LIB = os.path.join(HERE, "libpa_probes.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep hand-scheduled fp32 math scalar: no packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    # float32 divisions (quantisation scales) round correctly, as IEEE binary32
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


# per-source extra flags: the prefill kernel keeps MFMA accumulators in VGPRs
# (the softmax rescales them with vector ALU ops between MFMAs)
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    sub = os.path.basename(os.path.dirname(src))
    obj = os.path.join(BUILD, f"{sub}_{os.path.basename(src)}.o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PROBES, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBES_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources, {PROBES_LIB} from {len(probe_srcs)}")
    return LIB


if __name__ == "__main__":
    build()
