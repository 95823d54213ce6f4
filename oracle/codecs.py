"""Element codecs for the oracle (test infrastructure only).

bfloat16: the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent,
7 mantissa bits), so decoding is a 16-bit left shift.

FP8 E4M3 ("e4m3fn" in the OCP 8-bit floating point specification): 1 sign,
4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds subnormals
m * 2^-9; the code with all exponent and mantissa bits set (0x7F / 0xFF) is
NaN; there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
The pages ask only for "FP8" KV caches (KV-cache optimisation articles on the
"PagedAttention" tag page: FP8 halves the cache and is nearly lossless); this
format and a per-tensor scale are the reading taken.

Encoding rule (the reading used by the whole path): multiply by the
per-tensor inverse scale in float32, clamp the magnitude to 448 (saturate
finite; infinities saturate too), then round to the nearest representable
value with ties to even.  NaN encodes as 0x7F whatever its sign.

INT8: the KV-quantisation section of "From PagedAttention to Chunked
Prefill" (5.4) names FP16 -> INT8 as the standard step; the reading taken
is symmetric 8-bit integers with a per-tensor scale, like FP8 above: the
code is the float32 product x * (1 / scale) rounded to the nearest integer
(ties to even) and clamped to [-127, 127]; NaN encodes as 0; the value of a
code is code * scale.

INT4: the same section names 4-bit KV caches with KIVI's grouping -- keys
quantised along the channel (head_dim) axis, values along the token axis.
The reading taken: symmetric 4-bit integers in [-7, 7] (round half to even,
clamp, NaN -> 0, as for INT8); a key element uses its channel's scale (one
per KV head and channel, given by the caller); a value element uses its
token's scale (one per token and KV head, amax of the row / 7, computed when
the token is appended).  Storage: two codes per byte, element 2i in the low
nibble and 2i + 1 in the high nibble, each nibble sign-magnitude
(8 * [c < 0] + |c|); the nibble 8 (a negative zero) decodes to 0.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_decode(codes) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return c.view(np.float32).astype(np.float64)


def f32_decode(codes) -> np.ndarray:
    """uint32 binary32 bit patterns -> float64 (exact)."""
    with np.errstate(invalid="ignore"):
        return np.asarray(codes, dtype=np.uint32).view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * m * 2.0 ** -9             # subnormal
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 e4m3 codes -> float64 (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> uint8 e4m3 codes (saturate finite, round half to even).

    Works in float64, where every step below is exact: the magnitude is
    clamped, its binade exponent e is found (never below -6, the smallest
    normal exponent, so subnormals share the 2^-9 quantum), the value is
    divided by the quantum 2^(e-3) of that binade and rounded half-to-even to
    an integer r in [0, 16]; the code is (e + 7) * 8 + (r - 8), which also
    covers r = 16 (carry into the next binade) and the subnormals (e = -6).
    """
    x = np.asarray(x, dtype=np.float32)
    neg = np.signbit(x)
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.where(a == 0.0, -6, np.maximum(ex - 1, -6))
    quantum = np.ldexp(1.0, e - 3)
    r = np.rint(a / quantum)                  # IEEE round-half-even
    code = ((e + 7) * 8 + r - 8).astype(np.int64)
    out = (code.astype(np.uint8)) | (neg.astype(np.uint8) << np.uint8(7))
    out = np.where(nan, np.uint8(0x7F), out).astype(np.uint8)
    return out


def int8_decode(codes) -> np.ndarray:
    """Signed 8-bit codes (stored as uint8 bytes) -> float64 integers."""
    return np.asarray(codes, dtype=np.uint8).view(np.int8).astype(np.float64)


def int8_encode(x) -> np.ndarray:
    """float32 values -> uint8 bytes of int8 codes: rint (ties to even), clamp to
    [-127, 127], NaN -> 0."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    c = np.clip(np.rint(np.where(nan, 0.0, x)), -127.0, 127.0)   # +-inf clamp too
    return c.astype(np.int8).view(np.uint8)


def int4_encode(x) -> np.ndarray:
    """float32 values -> int8 arrays of 4-bit codes: rint (ties to even), clamp to
    [-7, 7], NaN -> 0."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    return np.clip(np.rint(np.where(nan, 0.0, x)), -7.0, 7.0).astype(np.int8)


def int4_pack(codes) -> np.ndarray:
    """4-bit codes [..., n] (n even) -> bytes [..., n / 2], sign-magnitude nibbles,
    element 2i low, 2i + 1 high."""
    c = np.asarray(codes, dtype=np.int64)
    nib = np.where(c < 0, 8, 0) + np.abs(c)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def int4_unpack(packed) -> np.ndarray:
    """Bytes [..., n / 2] -> int codes [..., n] (float64), inverse of int4_pack."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    nib = np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    mag = (nib & 7).astype(np.float64)
    return np.where(nib & 8, -mag, mag)


def int4_token_scale(rows) -> tuple[np.ndarray, np.ndarray]:
    """Per-row (token, head) scale of an INT4 value row and its float32 inverse:
    sigma = amax / 7 (NaN elements ignored; one float32 division), inv = 1 / sigma
    (one float32 division; inf for an all-zero row)."""
    x = np.abs(np.asarray(rows, dtype=np.float32))
    a = np.max(np.where(np.isnan(x), np.float32(0), x), axis=-1).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        sigma = (a / np.float32(7.0)).astype(np.float32)
        inv = (np.float32(1.0) / sigma).astype(np.float32)
    return sigma, inv


def f32_inverse(scale: float) -> np.float32:
    """Per-tensor inverse scale, one IEEE binary32 division."""
    return np.float32(1.0) / np.float32(scale)


def decode(codes, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Raw codes of a cache/query dtype -> float64 values (times ``scale`` for fp8)."""
    if dtype == "f32":
        return f32_decode(codes)
    if dtype == "bf16":
        return bf16_decode(codes)
    if dtype == "fp8":
        return e4m3_decode(codes) * np.float64(np.float32(scale))
    if dtype == "int8":
        return int8_decode(codes) * np.float64(np.float32(scale))
    raise ValueError(dtype)
