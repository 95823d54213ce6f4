"""Pins of the oracle's codecs against the format definitions and torch's CPU casts."""
import numpy as np
import pytest
import torch

from oracle import codecs, paged


def test_e4m3_table_known_values():
    t = codecs.E4M3_TABLE
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0
    assert t[0x3C] == 1.5
    assert t[0x40] == 2.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254


def test_e4m3_table_matches_torch_decode():
    allc = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = allc.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(tv), np.isnan(codecs.E4M3_TABLE))
    ok = ~np.isnan(tv)
    np.testing.assert_array_equal(tv[ok], codecs.E4M3_TABLE[ok])


def test_e4m3_roundtrip_all_finite_codes():
    c = np.arange(256, dtype=np.uint8)
    fin = np.isfinite(codecs.E4M3_TABLE)
    back = codecs.e4m3_encode(codecs.E4M3_TABLE[fin].astype(np.float32))
    np.testing.assert_array_equal(back, c[fin])


def test_e4m3_midpoints_round_half_to_even():
    t = codecs.E4M3_TABLE
    for c in range(0, 0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)            # exact in float32
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert codecs.e4m3_encode(mid) == even, hex(c)
        assert codecs.e4m3_encode(-mid) == even | 0x80
        above = np.nextafter(mid, np.float32(np.inf))
        below = np.nextafter(mid, np.float32(0))
        assert codecs.e4m3_encode(above) == c + 1
        assert codecs.e4m3_encode(below) == c


def test_e4m3_saturation_and_specials():
    v = np.array([448, 449, 463.99, 464, 464.01, 480, 1e6, np.inf, 3e38], np.float32)
    np.testing.assert_array_equal(codecs.e4m3_encode(v), 0x7E)
    np.testing.assert_array_equal(codecs.e4m3_encode(-v), 0xFE)
    assert codecs.e4m3_encode(np.float32(np.nan)) == 0x7F
    assert codecs.e4m3_encode(-np.float32(np.nan)) == 0x7F
    assert codecs.e4m3_encode(np.float32(0.0)) == 0x00
    assert codecs.e4m3_encode(np.float32(-0.0)) == 0x80
    tiny = np.array([2.0 ** -11, 2.0 ** -10, 1e-30, 1e-45], np.float32)   # below half the min subnormal, or exactly half
    np.testing.assert_array_equal(codecs.e4m3_encode(tiny), 0)
    assert codecs.e4m3_encode(np.float32(2.0 ** -10 * 1.0001)) == 1


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 10,
        rng.uniform(-448, 448, 200000),
        rng.standard_normal(50000) * 0.01,
        (codecs.E4M3_TABLE[np.isfinite(codecs.E4M3_TABLE)][:-1]),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    tc = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codecs.e4m3_encode(x), tc)


def test_fp8_append_multiplies_by_float32_inverse():
    scale = 0.0123
    inv = codecs.f32_inverse(scale)
    assert inv.dtype == np.float32 and inv == np.float32(1) / np.float32(scale)
    x = np.array([1.0, -2.5, 0.1], np.float32)
    got = paged.encode_tokens(x.view(np.uint32), "f32", "fp8", scale)
    np.testing.assert_array_equal(got, codecs.e4m3_encode((x * inv).astype(np.float32)))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 65536, 100000).astype(np.uint16)
    tv = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.bf16_decode(c)
    np.testing.assert_array_equal(np.isnan(tv), np.isnan(got))
    ok = ~np.isnan(tv)
    np.testing.assert_array_equal(tv[ok], got[ok])
    assert codecs.bf16_decode(np.uint16(0x3F80)) == 1.0
    assert codecs.bf16_decode(np.uint16(0xC000)) == -2.0


# ---- INT8 (symmetric, per-tensor scale) --------------------------------------------

def test_int8_decode_is_twos_complement():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b.copy()).view(torch.int8).numpy().astype(np.float64)
    assert np.array_equal(codecs.int8_decode(b), want)


def test_int8_integers_round_trip():
    x = np.arange(-127, 128, dtype=np.float32)
    assert np.array_equal(codecs.int8_decode(codecs.int8_encode(x)), x.astype(np.float64))


def test_int8_ties_to_even_and_saturation():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.49, 127.5, 1e9, -1e9,
                  np.inf, -np.inf, np.nan, -0.0], np.float32)
    want = np.array([0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127, 127, -127, 0, 0], np.float64)
    assert np.array_equal(codecs.int8_decode(codecs.int8_encode(x)), want)


def test_int8_encode_matches_torch_round_and_clamp():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(100000) * 80).astype(np.float32)
    t = torch.from_numpy(x).round().clamp(-127, 127).to(torch.int8).view(torch.uint8).numpy()
    assert np.array_equal(codecs.int8_encode(x), t)


def test_int8_cache_decodes_like_its_dequantised_f32_cache():
    """Attention over an int8 cache with scale 2^-4 equals attention over the f32 cache
    holding code * 2^-4 (exact in f32), through the oracle's decode path."""
    from oracle import paged
    rng = np.random.default_rng(4)
    bs, nkv, hd, nb = 4, 2, 8, 6
    kc = rng.integers(-127, 128, size=(nb, bs, nkv, hd)).astype(np.int8).view(np.uint8)
    vc = rng.integers(-127, 128, size=(nb, bs, nkv, hd)).astype(np.int8).view(np.uint8)
    sc = 2.0 ** -4
    kf = (kc.view(np.int8).astype(np.float32) * np.float32(sc)).view(np.uint32)
    vf = (vc.view(np.int8).astype(np.float32) * np.float32(sc)).view(np.uint32)
    q = rng.standard_normal((2, 2 * nkv, hd)).astype(np.float32).view(np.uint32)
    tables = np.array([[3, 0, 5], [1, 4, -1]])
    ctx = np.array([11, 6])
    a = paged.decode(q, "f32", kc, vc, "int8", tables, ctx, bs, 2, 0.3, sc, sc)
    b = paged.decode(q, "f32", kf, vf, "f32", tables, ctx, bs, 2, 0.3)
    assert np.array_equal(a, b)
