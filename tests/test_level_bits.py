"""The kernels take a delta's level rint(u) clamped to [-32, 31] from the bits
of the binary32 sum u + 1.5 * 2^23, clamped to [0x4B400000 - 32,
0x4B400000 + 31] (csrc/cg_build.h, level_bits; the histogram and the encoder
both use it), and the encoder takes the anchor's code rint(x inv_a) clamped to
[-127, 127] the same way with the bounds 0x4B400000 -+ 127 (anchor_bits).  The
oracle takes both the plain way, rint then clamp, and the two must agree for
every binary32 u.  This checks the identity on the CPU in binary32 arithmetic:
exhaustively around every half-integer tie in range, over a sweep of magnitudes
from subnormals to the largest finite values, and at the infinities."""
import pytest
import numpy as np

MAGIC = 0x4B400000


# (lowest, highest) code: the delta levels and the anchor codes
RANGES = [(-32, 31), (-127, 127)]


def level_plain(u, lo, hi):
    return np.clip(np.rint(u), lo, hi).astype(np.int64)


def level_bits(u, lo, hi):
    y = (u.astype(np.float32) + np.float32(12582912.0)).astype(np.float32)
    b = y.view(np.int32).astype(np.int64)
    return np.clip(b, MAGIC + lo, MAGIC + hi) - MAGIC


def check(u, lo, hi):
    u = np.asarray(u, dtype=np.float32)
    a, b = level_plain(u, lo, hi), level_bits(u, lo, hi)
    bad = np.nonzero(a != b)[0]
    assert bad.size == 0, (u[bad[:5]], a[bad[:5]], b[bad[:5]])
    # the low byte of the clamped bits is the code's two's-complement byte
    y = (u + np.float32(12582912.0)).astype(np.float32).view(np.int32).astype(np.int64)
    byte = np.clip(y, MAGIC + lo, MAGIC + hi) & 0xFF
    assert np.array_equal(byte, a & 0xFF)


@pytest.mark.parametrize("lo,hi", RANGES)
def test_ties_and_their_neighbours(lo, hi):
    # every x.5 in [-140, 140] and the 64 binary32 values on each side of it
    ties = np.arange(-280, 281, dtype=np.float32) / np.float32(2)
    bits = ties.view(np.int32)
    # neighbours by bit pattern, on the right side of zero for each sign
    offs = np.arange(-64, 65, dtype=np.int32)
    nb = (bits[:, None] + offs[None, :]).ravel().view(np.float32)
    check(np.concatenate([ties, nb[np.isfinite(nb)]]), lo, hi)


@pytest.mark.parametrize("lo,hi", RANGES)
def test_magnitude_sweep(lo, hi):
    rng = np.random.default_rng(7)
    exps = rng.integers(-149, 128, size=400000)
    mant = rng.random(400000) + 1.0
    u = (np.ldexp(mant, exps) * rng.choice([-1.0, 1.0], size=400000)).astype(np.float32)
    u = u[np.isfinite(u)]
    check(u, lo, hi)
    # the ends of the exact range, 2^22, and beyond
    edge = np.float32(2.0 ** 22)
    e = np.array([edge, -edge, np.nextafter(edge, np.float32(0)), np.nextafter(-edge, np.float32(0)),
                  np.float32(2.0 ** 23), np.float32(-(2.0 ** 23)), np.float32(1.5 * 2 ** 23),
                  np.float32(-1.5 * 2 ** 23), np.float32(3.0e38), np.float32(-3.0e38)], dtype=np.float32)
    check(e, lo, hi)


@pytest.mark.parametrize("lo,hi", RANGES)
def test_infinities_and_zeros(lo, hi):
    check(np.array([np.inf, -np.inf, 0.0, -0.0, np.float32(1e-45), np.float32(-1e-45)],
                   dtype=np.float32), lo, hi)
