"""Worker side of the exhaustive encoder sweep: the oracle's encoder on a range of
fp32 bit patterns.  Imports only numpy and the oracle, so spawned workers start fast."""
from __future__ import annotations

import numpy as np


def encode_range(args):
    """oracle.paged.encode_tokens of the patterns [start, start + n) (fp32 sources,
    per-tensor scale 1) as uint8 codes."""
    codec, start, n = args
    from oracle import paged
    x = (np.arange(n, dtype=np.uint64) + np.uint64(start)).astype(np.uint32)
    with np.errstate(invalid="ignore", over="ignore"):
        return paged.encode_tokens(x, "f32", codec, 1.0)
