"""Pins of the oracle's bandwidth-adaptive version choice (CacheGen blog, section
2.2) and of the simulated link: closed-form cases, monotonicity, and a link
whose transfer times are known exactly.  CPU only."""
import math

import numpy as np
import pytest

from oracle.controller import H, L, M, choose_version, stream_context
from synth.netsim import Link, bandwidth_trace

SIZES = [300_000, 200_000, 100_000]   # bytes left at H, M, L
DEC = [3.0, 2.0, 1.0]                 # ms of decoding left


def test_ample_bandwidth_takes_the_highest_quality():
    q, s = choose_version(1000.0, 1e9, SIZES, DEC)
    assert q == H and all(x > 1 for x in s)


def test_a_version_that_just_fits_is_taken():
    # H needs exactly the budget: 300_000 B at 1000 B/ms = 300 ms + 3 ms decoding
    q, s = choose_version(303.0, 1000.0, SIZES, DEC)
    assert q == H and s[H] == 1.0
    # a hair less and H no longer fits; M (200 + 2 ms) does
    q, s = choose_version(302.999, 1000.0, SIZES, DEC)
    assert q == M and s[H] < 1.0 <= s[M]


def test_scores_are_time_left_over_transfer_time():
    q, s = choose_version(150.0, 1000.0, SIZES, DEC)
    assert s == [(150.0 - 3.0) / 300.0, (150.0 - 2.0) / 200.0, (150.0 - 1.0) / 100.0]
    assert q == L


def test_nothing_fits_takes_the_version_done_soonest():
    # 100 ms of budget: none fits; L ends first (100 + 1 ms)
    q, _ = choose_version(50.0, 1000.0, SIZES, DEC)
    assert q == L
    # an overrun context (negative budget) still takes the version done soonest,
    # not the largest one a literal argmax of negative scores would pick
    q, s = choose_version(-40.0, 1000.0, SIZES, DEC)
    assert q == L and s[H] > s[L]
    # decoding can make a larger version end sooner
    q, _ = choose_version(10.0, 1000.0, [300_000, 200_000, 100_000], [0.0, 0.0, 500.0])
    assert q == M


def test_missing_versions_are_skipped():
    q, s = choose_version(1000.0, 1e9, [0, 200_000, 100_000], DEC)
    assert q == M and s[H] == 0.0
    q, _ = choose_version(1.0, 1.0, [0, 0, 100_000], DEC)
    assert q == L
    with pytest.raises(ValueError):
        choose_version(1.0, 1.0, [0, 0, 0], DEC)


@pytest.mark.parametrize("bad", [0.0, -1.0, math.inf, math.nan])
def test_bad_bandwidth_is_rejected(bad):
    with pytest.raises(ValueError):
        choose_version(10.0, bad, SIZES, DEC)


def test_more_bandwidth_or_budget_never_lowers_the_quality():
    rng = np.random.default_rng(7)
    for _ in range(300):
        size_l = int(rng.integers(1, 10**7))
        sizes = [int(size_l * rng.uniform(1.5, 3.0)), int(size_l * rng.uniform(1.0, 1.5)), size_l]
        sizes[1] = max(sizes[1], size_l)
        sizes[0] = max(sizes[0], sizes[1])
        dec = list(rng.uniform(0, 5, 3))
        budget = float(rng.uniform(-100, 3000))
        bws = np.sort(rng.uniform(1.0, 1e5, 12))
        qs = [choose_version(budget, b, sizes, dec)[0] for b in bws]
        assert all(a >= b for a, b in zip(qs, qs[1:])), (sizes, dec, budget, qs)
        budgets = np.sort(rng.uniform(-100, 5000, 12))
        qs = [choose_version(float(x), float(bws[5]), sizes, dec)[0] for x in budgets]
        assert all(a >= b for a, b in zip(qs, qs[1:])), (sizes, dec, qs)


def test_link_transfer_times_are_exact_on_a_known_trace():
    # 1 Gbit/s for one 10 ms step, then 2 Gbit/s: 125 and 250 bytes per microsecond
    link = Link(np.array([1.0, 2.0, 2.0]), step_ms=10.0)
    assert link.send(125_000 * 4) == pytest.approx(4.0)        # 4 ms at 1 Gbit/s
    assert link.send(125_000 * 6 + 250_000 * 5) == pytest.approx(11.0)  # 6 ms + 5 ms
    assert link.now == pytest.approx(15.0)
    with pytest.raises(ValueError):
        link.send(10**12)


def test_trace_mean_and_floor():
    g = bandwidth_trace(3, 200_000)
    assert g.min() >= 0.2
    assert abs(g.mean() - 3.0) < 0.1  # the log-normal correction keeps the mean
    assert np.array_equal(g, bandwidth_trace(3, 200_000))


def test_fixed_versions_and_adaptive_on_a_steady_link():
    sizes = [[300_000, 200_000, 100_000]] * 4
    dec = [[1.0, 1.0, 1.0]] * 4
    # 1000 B/ms steady: H takes 1200 ms + 1 ms of decoding
    for pol, ms in (("H", 1201.0), ("M", 801.0), ("L", 401.0)):
        link = Link(np.full(100, 8.0 * 1000 * 1e3 / 1e9), step_ms=100.0)
        t, vs, _ = stream_context(sizes, dec, 10_000.0, link.send, 1000.0, pol)
        assert t == pytest.approx(ms) and vs == ["HML".index(pol)] * 4
    # a 900 ms objective: the controller sends what fits and stays within it
    link = Link(np.full(100, 8.0 * 1000 * 1e3 / 1e9), step_ms=100.0)
    t, vs, _ = stream_context(sizes, dec, 900.0, link.send, 1000.0)
    assert t <= 900.0 and vs[0] == M
