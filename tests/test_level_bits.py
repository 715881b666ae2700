"""The kernels take a delta's level rint(u) clamped to [-32, 31] from the bits
of the binary32 sum u + 1.5 * 2^23, clamped to [0x4B400000 - 32,
0x4B400000 + 31] (csrc/cg_build.h, level_bits; the histogram and the encoder
both use it).  The oracle takes it the plain way, rint then clamp, and the two
must agree for every binary32 u.  This checks the identity on the CPU in
binary32 arithmetic: exhaustively around every half-integer tie in range, over
a sweep of magnitudes from subnormals to the largest finite values, and at the
infinities."""
import numpy as np

MAGIC = 0x4B400000


def level_plain(u):
    return np.clip(np.rint(u), -32, 31).astype(np.int64)


def level_bits(u):
    y = (u.astype(np.float32) + np.float32(12582912.0)).astype(np.float32)
    b = y.view(np.int32).astype(np.int64)
    return np.clip(b, MAGIC - 32, MAGIC + 31) - MAGIC


def check(u):
    u = np.asarray(u, dtype=np.float32)
    a, b = level_plain(u), level_bits(u)
    bad = np.nonzero(a != b)[0]
    assert bad.size == 0, (u[bad[:5]], a[bad[:5]], b[bad[:5]])


def test_ties_and_their_neighbours():
    # every x.5 in [-40, 40] and the 64 binary32 values on each side of it
    ties = np.arange(-80, 81, dtype=np.float32) / np.float32(2)
    bits = ties.view(np.int32)
    # neighbours by bit pattern, on the right side of zero for each sign
    offs = np.arange(-64, 65, dtype=np.int32)
    nb = (bits[:, None] + offs[None, :]).ravel().view(np.float32)
    check(np.concatenate([ties, nb[np.isfinite(nb)]]))


def test_magnitude_sweep():
    rng = np.random.default_rng(7)
    exps = rng.integers(-149, 128, size=400000)
    mant = rng.random(400000) + 1.0
    u = (np.ldexp(mant, exps) * rng.choice([-1.0, 1.0], size=400000)).astype(np.float32)
    u = u[np.isfinite(u)]
    check(u)
    # the ends of the exact range, 2^22, and beyond
    edge = np.float32(2.0 ** 22)
    e = np.array([edge, -edge, np.nextafter(edge, np.float32(0)), np.nextafter(-edge, np.float32(0)),
                  np.float32(2.0 ** 23), np.float32(-(2.0 ** 23)), np.float32(1.5 * 2 ** 23),
                  np.float32(-1.5 * 2 ** 23), np.float32(3.0e38), np.float32(-3.0e38)], dtype=np.float32)
    check(e)


def test_infinities_and_zeros():
    check(np.array([np.inf, -np.inf, 0.0, -0.0, np.float32(1e-45), np.float32(-1e-45)],
                   dtype=np.float32))
