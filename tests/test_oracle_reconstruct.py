"""Pins the oracle's reconstruction of delta tokens: the binary16 value nearest
to the exact real number ahat + (s - 32) * step, ties to even (CacheGen blog,
section 2.1: a delta token is the quantised anchor plus its coded delta).

The reference is exact rational arithmetic (fractions.Fraction) and a search
over neighbouring binary16 values: no binary64 rounding, no shared code.  The
cases cover what a plausible mistake would get wrong: the plain random case,
sums that land on a binary16 midpoint up to a tiny remainder of either sign
(where rounding through binary32 first goes wrong), exact midpoints (ties to
even), binary16 subnormals, the overflow threshold, and s = 32, where the
result is numpy's binary32 -> binary16 conversion of ahat."""
from fractions import Fraction

import numpy as np
import pytest

import synth

FINITE = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)


def nearest_f16_bits(x: Fraction) -> int:
    """Bits of the binary16 nearest to x (ties to even), by exact comparison
    with the neighbouring finite magnitudes; past 65504's half-way, infinity."""
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    if a >= Fraction(65520):
        return sign | 0x7C00
    i = int(np.searchsorted(FINITE, float(a)))
    best = None
    for j in range(max(0, i - 2), min(len(FINITE), i + 3)):
        d = abs(Fraction(FINITE[j]) - a)
        key = (d, j & 1)
        if best is None or key < best[0]:
            best = (key, j)
    return sign | best[1]


def exact(s, step, ahat):
    return [nearest_f16_bits(Fraction(float(a)) + (int(q) - 32) * Fraction(float(st)))
            for q, st, a in zip(s, step, ahat)]


def cases(n=4000, seed=5):
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 64, n).astype(np.uint8)
    step = (np.exp(rng.normal(-1.0, 2.0, n))).astype(np.float32)
    ahat = (rng.integers(-127, 128, n) * np.exp(rng.normal(-4.0, 2.0, n))).astype(np.float32)
    return s, step, ahat


def midpoint_cases(n=3000, seed=6):
    """ahat a binary16 midpoint (exact in binary32), the delta a tiny multiple of
    a step far below a binary32 ulp of ahat: binary32 rounding of the sum lands
    on the midpoint, the exact sum does not."""
    rng = np.random.default_rng(seed)
    h = rng.integers(0x0001, 0x7BFF, n).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2) * np.where(rng.random(n) < 0.5, -1.0, 1.0)
    ahat = mid.astype(np.float32)
    assert np.array_equal(ahat.astype(np.float64), mid)
    s = rng.choice(np.array([0, 31, 33, 63, 29, 40], np.uint8), n)
    step = (np.abs(mid) * 2.0 ** -40 * (0.5 + rng.random(n)) + 2.0 ** -120).astype(np.float32)
    return s, step, ahat


def test_random_triples_match_exact_rounding(oracle_lib):
    s, step, ahat = cases()
    assert list(oracle_lib.dequant_delta(s, step, ahat)) == exact(s, step, ahat)


def test_near_midpoints_follow_the_exact_sum(oracle_lib):
    s, step, ahat = midpoint_cases()
    got = oracle_lib.dequant_delta(s, step, ahat)
    assert list(got) == exact(s, step, ahat)
    # rounding through binary32 would give the tie's even neighbour instead in
    # about half of these: the cases do separate the two definitions
    via32 = (ahat + (s.astype(np.float32) - 32) * step).astype(np.float16).view(np.uint16)
    assert np.mean(via32 != got) > 0.3


def test_exact_midpoints_tie_to_even(oracle_lib):
    # ahat = 1, step = 2^-12: above 1 the binary16 spacing is 2^-10, so
    # 1 + k 2^-12 is a midpoint for k = 2 mod 4; below 1 the spacing is 2^-11
    # and 1 + k 2^-12 is a midpoint for odd negative k
    k = np.arange(-32, 32)
    s = (k + 32).astype(np.uint8)
    got = oracle_lib.dequant_delta(s, np.float32(2.0 ** -12), np.float32(1.0))
    assert list(got) == exact(s, np.full(64, 2.0 ** -12, np.float32), np.ones(64, np.float32))
    h = lambda x: int(np.float16(x).view(np.uint16))
    assert got[32 + 1] == h(1.0)                        # below the midpoint
    assert got[32 + 2] == h(1.0)                        # tie: 1 (even) beats 1 + 2^-10
    assert got[32 + 3] == h(1.0 + 2.0 ** -10)           # above it
    assert got[32 + 6] == h(1.0 + 2.0 ** -9)            # tie: the even neighbour above
    assert got[32 - 1] == h(1.0)                        # tie below 1: 1 (even)
    assert got[32 - 3] == h(1.0 - 2.0 ** -10)           # tie: 1 - 2^-10 (even)


def test_subnormal_and_overflow_results(oracle_lib):
    rng = np.random.default_rng(8)
    n = 2000
    s = rng.integers(0, 64, n).astype(np.uint8)
    step = (np.abs(rng.normal(0, 1, n)) * 2.0 ** -20).astype(np.float32)
    ahat = (rng.normal(0, 1, n) * 2.0 ** -16).astype(np.float32)
    got = oracle_lib.dequant_delta(s, step, ahat)
    assert list(got) == exact(s, step, ahat)
    assert np.mean((got & 0x7C00) == 0) > 0.5  # mostly binary16 subnormals
    # around the largest finite value 65504: 65504 + k; 65520 is the half-way
    # point to 2^16, a tie that goes to the even 2^16, i.e. infinity
    s2 = np.arange(64, dtype=np.uint8)
    st2 = np.full(64, 1.0, np.float32)
    a2 = np.full(64, 65504.0, np.float32)
    got2 = oracle_lib.dequant_delta(s2, st2, a2)
    assert list(got2) == exact(s2, st2, a2)
    assert got2[32 + 15] == 0x7BFF and got2[32 + 16] == 0x7C00 and got2[32 + 31] == 0x7C00
    assert got2[32 - 15] == 0x7BFF and got2[32 - 16] == 0x7BFE  # 65488: tie, even 65472


def test_zero_delta_is_the_binary32_to_binary16_conversion(oracle_lib):
    _, _, ahat = cases(20000, seed=9)
    step = np.full(ahat.shape, 0.37, np.float32)
    got = oracle_lib.dequant_delta(np.full(ahat.shape, 32, np.uint8), step, ahat)
    assert np.array_equal(got, ahat.astype(np.float16).view(np.uint16))


def test_decoded_deltas_are_the_exact_reconstruction(oracle_lib):
    """Every delta token the oracle's decoder writes is within one binary16 ulp
    of a binary64 evaluation of ahat + (s - 32) step (numpy's float64 -> float16
    conversion is correctly rounded), equal to it except on binary64 ties, and
    equal to the exact reconstruction on a sample."""
    w = synth.Workload("recon", layers=3, tokens=700, channels=64, seed=41, rho=0.85,
                       outlier_frac=0.03, chunk_tokens=256, group_tokens=10,
                       layer_group_end=(1, 2, 3), layer_step=(0.5, 1.0, 1.5),
                       qualities=(0, 1, 2))
    k, v = synth.gen_kv(w)
    t = oracle_lib.build_tables(oracle_lib.params_for(w), k, v)
    tv = oracle_lib.tables_view(t)
    rng = np.random.default_rng(1)
    for q in w.qualities:
        ko, vo = np.zeros_like(k), np.zeros_like(v)
        for ch in range(w.n_chunks):
            assert not oracle_lib.decode_blob(t, oracle_lib.encode_chunk(t, k, v, ch, q), ko, vo)
        for kv, y in enumerate((ko, vo)):
            anchors, syms = zip(*[oracle_lib.chunk_symbols(t, k, v, ch, q)
                                  for ch in range(w.n_chunks)])
            s = np.concatenate([sy[kv] for sy in syms], axis=1).astype(np.int64)  # [L, T, C]
            pos = np.arange(w.tokens) % w.chunk_tokens
            g_in_chunk = pos // w.group_tokens
            chunk = np.arange(w.tokens) // w.chunk_tokens
            a8 = np.stack([anchors[c][kv][:, g, :] for c, g in zip(chunk, g_in_chunk)], axis=1)
            sa = tv.scale_a[kv][:, None, :]
            ahat = (a8.astype(np.float32) * sa).astype(np.float32)
            step = np.broadcast_to(tv.step[q][kv][:, None, :], ahat.shape).astype(np.float32)
            is_delta = (pos % w.group_tokens != 0)[None, :, None] & np.ones_like(s, bool)
            y64 = (ahat.astype(np.float64) + (s - 32) * step.astype(np.float64)).astype(np.float16)
            yb = y.view(np.uint16)
            got = yb.view(np.float16).astype(np.float64)[is_delta]
            ref = y64.astype(np.float64)[is_delta]
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14))) - 10)
            assert np.all(np.abs(got - ref) <= ulp)
            assert np.mean(got == ref) > 0.9999
            idx = rng.choice(np.flatnonzero(is_delta.ravel()), 3000, replace=False)
            want = exact(s.ravel()[idx].astype(np.uint8), step.ravel()[idx], ahat.ravel()[idx])
            assert list(yb.ravel()[idx]) == want
