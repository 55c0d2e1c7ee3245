"""Pins for the oracle's IEEE binary16 codec (CPU only).

The codec is pinned to the IEEE 754 binary16 definition (closed-form bit
patterns), to exhaustive properties over all 65,536 patterns (round trip,
ties-to-even at every midpoint), and to NumPy's float16 conversions, which
are an independent implementation of the same definition.
"""
import numpy as np
import pytest

import oracle


def all_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_rounding_mode_is_nearest(oracle_lib):
    assert oracle_lib.oracle_rounding_mode_is_nearest() == 1


@pytest.mark.parametrize("bits,value", [
    (0x0000, 0.0), (0x3C00, 1.0), (0xBC00, -1.0), (0x4000, 2.0), (0xC000, -2.0), (0x3800, 0.5),
    (0x7BFF, 65504.0), (0x0400, 2.0 ** -14), (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24),
    (0x3555, 1365 * 2.0 ** -12), (0x6800, 2048.0), (0x6801, 2050.0), (0x7C00, np.inf), (0xFC00, -np.inf),
])
def test_decode_closed_forms(oracle_lib, bits, value):
    assert oracle_lib.oracle_f16_decode(bits) == value


def test_decode_negative_zero(oracle_lib):
    v = oracle_lib.oracle_f16_decode(0x8000)
    assert v == 0.0 and np.signbit(v)


def test_decode_exhaustive_matches_numpy():
    b = all_bits()
    got = oracle.f16_decode(b)
    ref = b.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_round_trip_exhaustive():
    b = all_bits()
    v = oracle.f16_decode(b)
    back = oracle.f16_encode(v)
    exp = (b >> 10) & 31
    frac = b & 1023
    is_nan = (exp == 31) & (frac != 0)
    assert np.array_equal(back[~is_nan], b[~is_nan])
    # NaN stays NaN (quiet, sign kept)
    nb = back[is_nan]
    assert np.all(((nb >> 10) & 31) == 31) and np.all((nb & 1023) != 0)
    assert np.array_equal(nb >> 15, b[is_nan] >> 15)


def test_ties_to_even_at_every_midpoint():
    """Every midpoint between adjacent finite fp16 values rounds to the
    neighbour whose last fraction bit is 0; a hair above or below rounds to
    the nearer neighbour."""
    b = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. 65504, increasing
    v = oracle.f16_decode(b)
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2  # exact in double
    got = oracle.f16_encode(mid)
    even = np.where((b[:-1] & 1) == 0, b[:-1], b[1:])
    assert np.array_equal(got, even)
    assert np.array_equal(oracle.f16_encode(np.nextafter(mid, -np.inf)), b[:-1])
    assert np.array_equal(oracle.f16_encode(np.nextafter(mid, np.inf)), b[1:])
    # negative side mirrors the positive side
    assert np.array_equal(oracle.f16_encode(-mid), even | 0x8000)


@pytest.mark.parametrize("x,bits", [
    (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (-65520.0, 0xFC00), (1e9, 0x7C00),
    (2049.0, 0x6800), (2051.0, 0x6802), (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002),
    (2.0 ** -24, 0x0001), (1023.5 * 2.0 ** -24, 0x0400), (1.0 + 2.0 ** -11, 0x3C00),
    (1.0 + 3 * 2.0 ** -11, 0x3C02), (np.inf, 0x7C00), (-np.inf, 0xFC00), (-0.0, 0x8000), (0.0, 0x0000),
    (1e-30, 0x0000), (-1e-30, 0x8000),
])
def test_encode_known_points(oracle_lib, x, bits):
    assert oracle_lib.oracle_f16_encode(x) == bits


def test_encode_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(12345)
    n = 1_000_000
    # log-uniform magnitudes over the whole fp16 range and a bit beyond, both signs
    mag = np.exp2(rng.uniform(-27, 17, n))
    x = np.where(rng.random(n) < 0.5, -mag, mag)
    got = oracle.f16_encode(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
