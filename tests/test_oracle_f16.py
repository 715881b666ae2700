"""Pins the oracle's IEEE binary16 conversions against numpy (an independent
implementation of the same standard)."""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_f16_to_f32_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_lib.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_roundtrip_of_every_half(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float32)
    fin = np.isfinite(vals)
    back = oracle_lib.f32_to_f16(vals[fin])
    assert np.array_equal(back, bits[fin])


def test_f32_to_f16_midpoints_tie_to_even(oracle_lib):
    # midpoints between consecutive positive finite halves are exact in binary32
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    ours = oracle_lib.f32_to_f16(np.concatenate([mid, -mid]))
    ref = np.concatenate([mid, -mid]).astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to the even significand
    even = np.where(bits % 2 == 0, bits, bits + 1)
    assert np.array_equal(ours[: bits.size], even)


def test_f32_to_f16_random_bit_patterns(oracle_lib):
    rng = np.random.default_rng(123)
    x = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    ours = oracle_lib.f32_to_f16(x)
    ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all(ours[nan] & 0x3FF)


def test_f32_to_f16_ranges(oracle_lib):
    rng = np.random.default_rng(7)
    # the magnitudes the codec produces: normal, subnormal and overflow boundaries
    x = np.concatenate([
        rng.standard_normal(500_000).astype(np.float32) * 10,
        (rng.standard_normal(200_000) * 1e-6).astype(np.float32),
        np.array([65504, 65519.996, 65520, 65536, 6.1035156e-05, 6.0975552e-05, 5.9604645e-08,
                  2.9802322e-08, 2.9802326e-08, 0.0, -0.0, np.inf, -np.inf], np.float32),
    ])
    assert np.array_equal(oracle_lib.f32_to_f16(x), x.astype(np.float16).view(np.uint16))
