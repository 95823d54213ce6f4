"""The C boundary without a GPU: exported symbols, binding signatures, host-side checks.

Every function declared in include/pa.h must be exported by libpa.so, the
Python binding must declare the same number of arguments as the header, and
the argument checks that run on the host before anything is enqueued must give
the documented statuses.  Nothing here launches a kernel: the calls below stop
at a host check (dummy pointers are used only where the header says the call
returns before any device work, and only when no GPU is visible).
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_cache_74_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(7)
F32, BF16, FP8 = pa.PA_F32, pa.PA_BF16, pa.PA_FP8_E4M3


def _declarations():
    """{name: number of parameters} of every function declared in pa.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(pa_\w+)\s*\(([^;{]*?)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail(f"{pa.LIB_PATH} is not built")
    return pa.lib()


def test_header_declares_the_boundary():
    decl = _declarations()
    for name in ("pa_kv_append", "pa_decode", "pa_prefill_chunk", "pa_slot_mapping",
                 "pa_decode_workspace_bytes", "pa_prefill_workspace_bytes",
                 "pa_decode_partials", "pa_decode_merge", "pa_status_string", "pa_abi_version"):
        assert name in decl, name


def test_every_declared_symbol_is_exported(lib):
    for name in _declarations():
        assert hasattr(lib, name), f"{name} declared in pa.h but not exported"


def test_no_undeclared_exports(lib):
    nm = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T pa_" in l}
    assert exported == set(_declarations()), exported ^ set(_declarations())


PROBES_HEADER = os.path.join(ROOT, "paged_kv_cache_74_amd", "probes", "pa_probes.h")


def test_measurement_probes_live_in_their_own_library():
    """libpa.so carries only the method; the benchmark's probes are libpa_probes.so."""
    from paged_kv_cache_74_amd import probes
    text = re.sub(r"/\*.*?\*/", "", open(PROBES_HEADER).read(), flags=re.S)
    declared = set(re.findall(r"\b(pa_\w+)\s*\(", text))
    assert declared == {"pa_ceiling_stream_read", "pa_ceiling_gather_read", "pa_ceiling_mfma_bf16",
                        "pa_ceiling_mfma_bf16_lds", "pa_probe_lds_pattern"}
    assert not declared & set(_declarations())
    nm = subprocess.run(["nm", "-D", "--defined-only", probes.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    assert {l.split()[-1] for l in nm.splitlines() if " T pa_" in l} == declared
    lp = probes.lib()
    assert all(hasattr(lp, n) for n in declared)


def test_binding_arity_matches_header(lib):
    for name, n in _declarations().items():
        f = getattr(lib, name)
        assert len(f.argtypes or []) == n, (name, len(f.argtypes or []), n)


def test_abi_version_and_status_strings(lib):
    assert lib.pa_abi_version() == 2
    names = [lib.pa_status_string(s).decode() for s in range(7)]
    assert len(set(names)) == 7 and all(names)
    assert lib.pa_status_string(99).decode()          # unknown codes still give text


# host-side checks that return before any device call ---------------------------------

def _append(lib, **kw):
    a = dict(k=None, v=None, cdt=BF16, nb=8, bs=16, nkv=2, hd=64, kn=None, vn=None, sdt=BF16,
             slots=None, n=4, ks=1.0, vs=1.0)
    a.update(kw)
    return lib.pa_kv_append(a["k"], a["v"], a["cdt"], a["nb"], a["bs"], a["nkv"], a["hd"],
                            a["kn"], a["vn"], a["sdt"], a["slots"], a["n"], a["ks"], a["vs"], None)


def test_kv_append_argument_checks(lib):
    assert _append(lib, n=0) == PA_OK                  # nothing to write: no pointer is read
    assert _append(lib, nb=-1) == PA_ERR_SHAPE
    assert _append(lib, bs=0) == PA_ERR_SHAPE
    assert _append(lib, n=-1) == PA_ERR_SHAPE
    assert _append(lib, hd=12) == PA_ERR_UNSUPPORTED   # rows move in 8-element chunks
    assert _append(lib) == PA_ERR_NULL


@pytest.mark.skipif(not _no_gpu(), reason="dummy pointers are passed only where no GPU is visible")
def test_kv_append_dtype_and_scale_checks(lib):
    d = dict(k=0x1000, v=0x1000, kn=0x1000, vn=0x1000, slots=0x1000)
    assert _append(lib, cdt=BF16, sdt=F32, **d) == PA_ERR_DTYPE
    assert _append(lib, cdt=F32, sdt=BF16, **d) == PA_ERR_DTYPE
    assert _append(lib, cdt=FP8, sdt=FP8, **d) == PA_ERR_DTYPE
    assert _append(lib, cdt=FP8, sdt=BF16, ks=0.0, **d) == PA_ERR_SHAPE
    assert _append(lib, cdt=FP8, sdt=BF16, vs=float("nan"), **d) == PA_ERR_SHAPE


def _decode(lib, **kw):
    a = dict(out=None, q=None, qdt=BF16, k=None, v=None, cdt=BF16, nb=8, bs=16, nkv=2, hd=128,
             g=4, tables=None, mb=4, ctx=None, ns=2, maxc=64, split=0)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["qdt"], a["k"], a["v"], a["cdt"], a["nb"], a["bs"],
                         a["nkv"], a["hd"], a["g"], a["tables"], a["mb"], a["ctx"], a["ns"],
                         a["maxc"], 0.1, 1.0, 1.0, a["split"], None, 0, None)


def test_decode_argument_checks(lib):
    assert _decode(lib, ns=0) == PA_OK
    assert _decode(lib, g=3) == PA_ERR_UNSUPPORTED
    assert _decode(lib, hd=96) == PA_ERR_UNSUPPORTED
    assert _decode(lib, bs=24) == PA_ERR_UNSUPPORTED
    assert _decode(lib, bs=512) == PA_ERR_UNSUPPORTED
    assert _decode(lib, nb=-1) == PA_ERR_SHAPE
    assert _decode(lib, qdt=F32, cdt=BF16) == PA_ERR_DTYPE
    assert _decode(lib, qdt=BF16, cdt=F32) == PA_ERR_DTYPE
    assert _decode(lib) == PA_ERR_NULL


def _prefill(lib, **kw):
    a = dict(out=None, q=None, qdt=BF16, cu=None, ns=2, tq=64, mq=32, k=None, v=None, cdt=BF16,
             nb=8, bs=16, nkv=2, hd=128, g=4, tables=None, mb=4, ctx=None, maxc=64, causal=1,
             scale=0.1)
    a.update(kw)
    return lib.pa_prefill_chunk(a["out"], a["q"], a["qdt"], a["cu"], a["ns"], a["tq"], a["mq"],
                                a["k"], a["v"], a["cdt"], a["nb"], a["bs"], a["nkv"], a["hd"],
                                a["g"], a["tables"], a["mb"], a["ctx"], a["maxc"], a["causal"],
                                a["scale"], 1.0, 1.0, None, 0, None)


def test_prefill_argument_checks(lib):
    assert _prefill(lib, ns=0) == PA_OK
    assert _prefill(lib, tq=0) == PA_OK
    assert _prefill(lib, hd=256) == PA_ERR_UNSUPPORTED
    assert _prefill(lib, g=16) == PA_ERR_UNSUPPORTED
    assert _prefill(lib, bs=3) == PA_ERR_UNSUPPORTED
    assert _prefill(lib, qdt=F32) == PA_ERR_DTYPE              # (F32, BF16)
    assert _prefill(lib, cdt=F32) == PA_ERR_DTYPE              # (BF16, F32)
    assert _prefill(lib, qdt=F32, cdt=FP8) == PA_ERR_DTYPE
    assert _prefill(lib, qdt=F32, cdt=F32) == PA_ERR_NULL      # (F32, F32) is supported
    assert _prefill(lib, ns=-1) == PA_ERR_SHAPE
    assert _prefill(lib) == PA_ERR_NULL


@pytest.mark.skipif(not _no_gpu(), reason="dummy pointers are passed only where no GPU is visible")
def test_prefill_scale_checks(lib):
    d = dict(out=0x1000, q=0x1000, cu=0x1000, k=0x1000, v=0x1000, tables=0x1000, ctx=0x1000)
    assert _prefill(lib, scale=0.0, **d) == PA_ERR_SHAPE
    assert _prefill(lib, scale=-0.1, **d) == PA_ERR_SHAPE
    assert _prefill(lib, scale=float("inf"), **d) == PA_ERR_SHAPE
    assert _prefill(lib, scale=float("nan"), **d) == PA_ERR_SHAPE
    assert _prefill(lib, qdt=F32, cdt=F32, scale=0.0, **d) == PA_ERR_SHAPE
    assert _prefill(lib, qdt=F32, cdt=F32, **d) == PA_ERR_WORKSPACE     # no workspace given
    assert lib.pa_prefill_workspace_bytes(2, 64, 32, 8, 2, 128, 64) > 0


def _copy(lib, **kw):
    a = dict(dk=None, dv=None, dn=8, sk=None, sv=None, sn=8, cdt=BF16, bs=16, nkv=2, hd=64,
             pairs=None, n=4)
    a.update(kw)
    return lib.pa_copy_blocks(a["dk"], a["dv"], a["dn"], a["sk"], a["sv"], a["sn"], a["cdt"],
                              a["bs"], a["nkv"], a["hd"], a["pairs"], a["n"], None)


def test_copy_blocks_argument_checks(lib):
    assert _copy(lib, n=0) == PA_OK
    assert _copy(lib, dn=-1) == PA_ERR_SHAPE
    assert _copy(lib, bs=0) == PA_ERR_SHAPE
    assert _copy(lib, n=-2) == PA_ERR_SHAPE
    assert _copy(lib, cdt=7) == PA_ERR_DTYPE
    assert _copy(lib, cdt=FP8, bs=1, nkv=1, hd=4) == PA_ERR_UNSUPPORTED   # 4-byte blocks
    assert _copy(lib) == PA_ERR_NULL


@pytest.mark.skipif(not _no_gpu(), reason="dummy pointers are passed only where no GPU is visible")
def test_copy_blocks_alignment_check(lib):
    d = dict(dk=0x1000, dv=0x1000, sk=0x1000, sv=0x1008, pairs=0x1000)
    assert _copy(lib, **d) == PA_ERR_SHAPE                                 # 16-byte blocks need 16


def test_int4_argument_checks(lib):
    INT4 = pa.PA_INT4
    app = lambda **kw: lib.pa_kv_append_int4(
        kw.get("k"), kw.get("v"), kw.get("vs"), kw.get("nb", 8), 16, 2, kw.get("hd", 64),
        kw.get("kn"), kw.get("vn"), kw.get("sdt", BF16), kw.get("slots"), kw.get("n", 4),
        kw.get("ks"), None)
    assert app(n=0) == PA_OK
    assert app(nb=-1) == PA_ERR_SHAPE
    assert app(hd=96) == PA_ERR_UNSUPPORTED
    assert app(sdt=FP8) == PA_ERR_DTYPE
    assert app() == PA_ERR_NULL
    # the per-tensor-scale entry points refuse an INT4 cache
    assert _decode(lib, cdt=INT4) == PA_ERR_DTYPE
    dec = lambda **kw: lib.pa_decode_int4(
        None, None, kw.get("qdt", BF16), None, None, None, None, 8, 16, 2, kw.get("hd", 128),
        kw.get("g", 4), None, 4, None, kw.get("ns", 2), 64, 0.1, 0, None, 0, None)
    assert dec(ns=0) == PA_OK
    assert dec(hd=96) == PA_ERR_UNSUPPORTED
    assert dec(qdt=F32) == PA_ERR_DTYPE
    assert dec() == PA_ERR_NULL
    assert _copy(lib, cdt=INT4, bs=1, nkv=1, hd=8) == PA_ERR_UNSUPPORTED   # 4-byte blocks
    assert _copy(lib, cdt=INT4) == PA_ERR_NULL


def test_decode_no_alloc_checks(lib):
    """Host checks of the allocation-free decode, before any HIP call."""
    call = lambda **kw: lib.pa_decode_no_alloc(
        None, None, BF16, None, None, kw.get("cdt", BF16), 8, 16, 8, 128, kw.get("g", 4), None,
        256, None, kw.get("ns", 2), kw.get("maxc", 4096), 0.1, 1.0, 1.0, 0, None)
    assert call(ns=0) == PA_OK
    assert call(g=3) == PA_ERR_UNSUPPORTED
    assert call(cdt=pa.PA_INT4) == PA_ERR_DTYPE
    assert call(ns=1 << 16) == PA_ERR_WORKSPACE           # partials beyond the fixed scratch
    assert pa.pa_decode_workspace_bytes(1 << 16, 32, 8, 128, 4096, 0) > pa.PA_NO_ALLOC_SCRATCH_BYTES
    # the binding's constant is the header's
    text = open(HEADER).read()
    assert "#define PA_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert pa.PA_NO_ALLOC_SCRATCH_BYTES == 64 << 20
