"""Binding of libpa_probes.so: measurement probes for the benchmark.

Not part of the paged attention library.  Each probe is a plain kernel that
reads whole pool blocks (in a given order) or a buffer contiguously, or only
issues bf16 MFMAs, so the benchmark can report what this GPU reaches for the
same bytes or the same instruction, or repeats one LDS access pattern for the
bank-conflict counter (declarations: probes/pa_probes.h).
Argument marshalling only, as in the main binding.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .. import PagedAttentionError, _dev, _need, _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "libpa_probes.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"probe library not built: {LIB_PATH} is missing "
                               "(run `python -m paged_kv_cache_74_amd.build`)")
        _lib = ctypes.CDLL(LIB_PATH)
        P, I, L64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        for name, args in (("pa_ceiling_stream_read", (P, L64, P, I, P)),
                           ("pa_ceiling_gather_read", (P, P, L64, I, P, L64, P, I, P)),
                           ("pa_ceiling_mfma_bf16", (P, I, I, P)),
                           ("pa_ceiling_mfma_bf16_lds", (P, I, I, P)),
                           ("pa_probe_lds_pattern", (P, I, I, P, I, P))):
            f = getattr(_lib, name)
            f.restype = ctypes.c_int
            f.argtypes = list(args)
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise PagedAttentionError(fn, status)


def pa_ceiling_stream_read(buf: torch.Tensor, sink: torch.Tensor, num_wgs: int,
                           stream=None) -> None:
    """Read all of buf once, contiguously; sink: 4-byte [4 * num_wgs]."""
    _dev(buf, sink)
    _need(sink.numel() >= 4 * num_wgs and sink.element_size() == 4,
          "sink: 4-byte [4 * num_wgs]")
    _check("pa_ceiling_stream_read", lib().pa_ceiling_stream_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), num_wgs, _stream(stream)))


def pa_ceiling_gather_read(k_pool: torch.Tensor, v_pool: torch.Tensor, blocks: torch.Tensor,
                           sink: torch.Tensor, num_wgs: int, stream=None) -> None:
    """Read whole pool blocks in list order."""
    _dev(k_pool, v_pool, blocks, sink)
    _need(k_pool.shape == v_pool.shape, "pools of one shape")
    _need(blocks.dtype == torch.int32 and sink.numel() >= 4 * num_wgs and
          sink.element_size() == 4, "blocks int32, sink 4-byte [4 * num_wgs]")
    nb = k_pool.shape[0]
    _check("pa_ceiling_gather_read", lib().pa_ceiling_gather_read(
        _ptr(k_pool), _ptr(v_pool), nb, k_pool.numel() * k_pool.element_size() // nb,
        _ptr(blocks), blocks.numel(), _ptr(sink), num_wgs, _stream(stream)))


def pa_ceiling_mfma_bf16(sink: torch.Tensor, num_wgs: int, iters: int, stream=None) -> None:
    """Matrix-core issue rate; sink: float32 [num_wgs * 4]."""
    _dev(sink)
    _need(sink.dtype == torch.float32 and sink.numel() >= 4 * num_wgs, "sink: float32 [4 W]")
    _check("pa_ceiling_mfma_bf16", lib().pa_ceiling_mfma_bf16(_ptr(sink), num_wgs, iters,
                                                              _stream(stream)))


def pa_ceiling_mfma_bf16_lds(sink: torch.Tensor, num_wgs: int, iters: int, stream=None) -> None:
    """Matrix-core issue rate with one operand read from LDS per MFMA; sink: float32 [num_wgs * 4]."""
    _dev(sink)
    _need(sink.dtype == torch.float32 and sink.numel() >= 4 * num_wgs, "sink: float32 [4 W]")
    _check("pa_ceiling_mfma_bf16_lds", lib().pa_ceiling_mfma_bf16_lds(_ptr(sink), num_wgs, iters,
                                                                      _stream(stream)))


LDS_KINDS = {"write_b128": 0, "read_b128": 1, "read_b64_tr_b16": 2, "read_b64": 3}


def pa_probe_lds_pattern(offsets: torch.Tensor, kind: str, iters: int, sink: torch.Tensor,
                         num_wgs: int, stream=None) -> None:
    """One LDS access pattern per launch; offsets: int32/uint32 [64] byte offsets per lane,
    sink: 4-byte [num_wgs]."""
    _dev(offsets, sink)
    _need(offsets.numel() == 64 and offsets.element_size() == 4, "offsets: 4-byte [64]")
    _need(sink.numel() >= num_wgs and sink.element_size() == 4, "sink: 4-byte [num_wgs]")
    _need(kind in LDS_KINDS, f"kind: one of {sorted(LDS_KINDS)}")
    _check("pa_probe_lds_pattern", lib().pa_probe_lds_pattern(
        _ptr(offsets), LDS_KINDS[kind], iters, _ptr(sink), num_wgs, _stream(stream)))
