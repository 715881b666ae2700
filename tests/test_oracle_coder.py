"""Pins the oracle's range coder without a second implementation of it:
brute force over every string on tiny alphabets (round trip, injectivity,
independence from the bytes that follow a stream), information-theoretic
length bounds derived from the coder's invariants, and closed forms."""
import itertools
import math

import numpy as np
import pytest

M = 1 << 15
# Per symbol the coder spends -log2(freq/2^15) plus at most log2(1 + 2^-9) bits
# (the range is truncated to a multiple of 2^15 of a value >= 2^24); the flush
# adds one or two bytes.  So  sum(cost) <= 8*len <= sum(cost) + 0.002815*n + 16.
SLACK_PER_SYMBOL = math.log2(1 + 2.0 ** -9)


def cost_bits(symbols, freq):
    f = np.asarray(freq, np.float64)
    return float(np.sum(-np.log2(f[np.asarray(symbols, np.int64)] / M))) if len(symbols) else 0.0


def tables_for(nsym, rng):
    if nsym == 1:
        return [np.array([M], np.uint16)]
    uni = np.full(nsym, M // nsym, np.uint16)
    uni[0] += M - int(uni.sum())
    extreme = np.ones(nsym, np.uint16)
    extreme[-1] = M - (nsym - 1)
    rand = rng.integers(1, 4000, nsym).astype(np.float64)
    rand = np.maximum(1, np.floor(rand / rand.sum() * (M - nsym))).astype(np.int64) + 0
    rand[np.argmax(rand)] += M - rand.sum()
    return [uni, extreme, rand.astype(np.uint16)]


def check_length(n, nbytes, cost):
    if n == 0:
        assert nbytes == 0
        return
    assert 8 * nbytes >= cost - 1e-9, (n, nbytes, cost)
    assert 8 * nbytes <= cost + SLACK_PER_SYMBOL * n + 16 + 1e-9, (n, nbytes, cost)


@pytest.mark.parametrize("nsym", [1, 2, 3, 4])
def test_bruteforce_all_strings(oracle_lib, nsym):
    rng = np.random.default_rng(nsym)
    maxlen = 8 if nsym <= 3 else 7
    for freq in tables_for(nsym, rng):
        for n in range(0, maxlen + 1):
            seen = {}
            for s in itertools.product(range(nsym), repeat=n):
                s = np.array(s, np.uint8)
                code = oracle_lib.rc_encode(s, freq)
                check_length(n, len(code), cost_bits(s, freq))
                # decodes with zeros, ones and random bytes after the stream
                for tail in (b"", b"\xff" * 8, rng.integers(0, 256, 8, dtype=np.uint8).tobytes()):
                    got, used, bad = oracle_lib.rc_decode(code + tail, n, freq)
                    assert np.array_equal(got, s) and not bad
                    if n:
                        # reads the four-byte window plus one byte per emitted byte
                        assert used <= len(code) + 3
                assert code not in seen, "two strings share a code"
                seen[code] = True


def test_single_symbol_alphabet_costs_one_byte(oracle_lib):
    for n in (1, 2, 100, 10000):
        code = oracle_lib.rc_encode(np.zeros(n, np.uint8), [M])
        assert len(code) == 1
    assert oracle_lib.rc_encode(np.zeros(0, np.uint8), [M]) == b""


@pytest.mark.parametrize("k", [1, 3, 6, 8])
def test_uniform_power_of_two_tables(oracle_lib, k):
    nsym = 1 << k
    freq = np.full(nsym, M // nsym, np.uint16)
    rng = np.random.default_rng(k)
    for n in (1, 17, 1000, 20000):
        s = rng.integers(0, nsym, n).astype(np.uint8)
        code = oracle_lib.rc_encode(s, freq)
        assert n * k <= 8 * len(code) <= n * k + SLACK_PER_SYMBOL * n + 16
        got, _, bad = oracle_lib.rc_decode(code, n, freq)
        assert np.array_equal(got, s) and not bad


def test_dominant_symbol_is_nearly_free(oracle_lib):
    freq = np.ones(64, np.uint16)
    freq[32] = M - 63
    for n in (10, 1000, 100000):
        code = oracle_lib.rc_encode(np.full(n, 32, np.uint8), freq)
        bits = n * -math.log2((M - 63) / M)
        assert len(code) <= 2 + math.ceil((bits + SLACK_PER_SYMBOL * n) / 8)


def test_long_random_strings_and_carries(oracle_lib):
    rng = np.random.default_rng(99)
    for trial in range(40):
        nsym = int(rng.integers(2, 65))
        # skewed tables put most mass at the top of the range, where carries happen
        w = rng.dirichlet(np.full(nsym, 0.3))
        f = np.maximum(1, np.floor(w * (M - nsym))).astype(np.int64)
        f[np.argmax(f)] += M - f.sum()
        f = f.astype(np.uint16)
        n = int(rng.integers(1, 60000))
        s = rng.choice(nsym, n, p=f / M).astype(np.uint8)
        code = oracle_lib.rc_encode(s, f)
        check_length(n, len(code), cost_bits(s, f))
        tail = rng.integers(0, 256, 8, dtype=np.uint8).tobytes()
        got, used, bad = oracle_lib.rc_decode(code + tail, n, f)
        assert np.array_equal(got, s) and not bad and used <= len(code) + 3


def test_codes_depend_on_every_symbol(oracle_lib):
    """Changing any one symbol of a string changes its code (a dropped or
    misplaced update in the coder would make some positions invisible)."""
    rng = np.random.default_rng(5)
    f = np.full(64, 512, np.uint16)
    s = rng.integers(0, 64, 300).astype(np.uint8)
    base = oracle_lib.rc_encode(s, f)
    for i in range(0, 300, 7):
        t = s.copy()
        t[i] = (t[i] + 1) % 64
        assert oracle_lib.rc_encode(t, f) != base
