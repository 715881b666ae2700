"""Pins the oracle's statistics and probability tables: the channel std against
numpy's std, the anchor scale against numpy's max, the normalisation by its
invariants and special cases, the layer-group steps against the constants the
pages print (tests/golden/pages_constants.json), the serialized layout by an
independent Python reader."""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M = 1 << 15


def test_normalize_invariants(oracle_lib):
    rng = np.random.default_rng(0)
    cases = [np.zeros(64), np.ones(64), np.full(64, 7), np.eye(64)[5] * 1000,
             np.eye(64)[63] * (2**32 - 1), rng.integers(0, 2**32, 64),
             rng.integers(0, 3, 64), np.r_[np.full(32, 10**9), np.zeros(32)]]
    cases += [rng.poisson(rng.gamma(0.5, 200, 64)) for _ in range(200)]
    for c in cases:
        c = np.asarray(c, np.uint64).astype(np.uint32)
        f = oracle_lib.normalize(c).astype(np.int64)
        assert f.sum() == M and f.min() >= 1
        N = int(c.astype(np.int64).sum())
        ci = c.astype(np.int64)
        # order-preserving: more counts never get fewer slots (the remainder only
        # goes to a most-counted symbol)
        levels = np.unique(ci)
        for lo, hi in zip(levels[:-1], levels[1:]):
            assert f[ci == lo].max() <= f[ci == hi].min()
        if N:
            exact = ci * (M - 64) / N
            extra = f - 1 - np.floor(exact)
            assert np.all((extra == 0) | (ci == ci.max()))
            assert 0 <= extra.sum() < 64


def test_normalize_special_cases(oracle_lib):
    assert np.all(oracle_lib.normalize(np.zeros(64, np.uint32)) == 512)
    assert np.all(oracle_lib.normalize(np.full(64, 3, np.uint32)) == 512)
    f = oracle_lib.normalize(np.eye(64, dtype=np.uint32)[17] * 12345)
    assert f[17] == M - 63 and np.all(np.delete(f, 17) == 1)
    # ties for the maximum go to the lowest index
    c = np.zeros(64, np.uint32)
    c[[3, 9, 20]] = 1
    f = oracle_lib.normalize(c)
    share = 1 + (M - 64) // 3            # 10902 each, one slot left over
    assert 61 + 3 * share == M - 1
    assert (f[3], f[9], f[20]) == (share + 1, share, share)


def test_channel_std_matches_numpy(oracle_lib):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((3, 777, 40)) * np.exp(rng.standard_normal(40))[None, None, :]
         + rng.standard_normal(40)[None, None, :] * 5).astype(np.float16)
    x[0, :, 0] = 1.5            # constant channel: no spread, reads as std 1
    x[1, :, 1] = 0.0            # all-zero channel
    x[2, 5, 2] = 60000.0        # large outlier
    x[2, :, 3] = np.float16(6e-8)  # subnormals
    sig, amax, nf = oracle_lib.channel_stats(x)
    assert not nf
    ref = x.astype(np.float64).std(axis=1)
    ref = np.where(ref == 0, 1.0, ref)
    assert np.allclose(sig, ref, rtol=1e-12, atol=0)
    assert np.array_equal(amax, np.abs(x.astype(np.float32)).max(axis=1))
    y = x.copy()
    y[1, 3, 4] = np.inf
    assert oracle_lib.channel_stats(y)[2]
    y = x.copy()
    y[0, 0, 0] = np.nan
    assert oracle_lib.channel_stats(y)[2]


def small_workload(**kw):
    base = dict(layers=4, tokens=700, channels=96, seed=21, rho=0.85, outlier_frac=0.05,
                chunk_tokens=256, group_tokens=10, layer_group_end=(1, 3, 4),
                layer_step=(0.5, 1.0, 1.5), qualities=(0, 1, 2))
    base.update(kw)
    return synth.Workload("small", **base)


def test_tables_layout_and_scales(oracle_lib):
    w = small_workload()
    k, v = synth.gen_kv(w)
    p = oracle_lib.params_for(w)
    t, counts = oracle_lib.build_tables(p, k, v, with_counts=True)
    tv = oracle_lib.tables_view(t)
    h = tv.header
    assert h["magic"] == b"CGT1" and h["prob_bits"] == 15 and h["n_symbols"] == 64
    assert (h["layers"], h["tokens"], h["channels"]) == (4, 700, 96)
    for kv, x in enumerate((k, v)):
        xd = x.astype(np.float64)
        sig = xd.std(axis=1)
        amax = np.abs(xd).max(axis=1)
        # anchor scale: absmax / 127, rounded once to binary32
        assert np.array_equal(tv.scale_a[kv], (amax / 127.0).astype(np.float32))
        assert np.array_equal(tv.inv_a[kv], (1.0 / tv.scale_a[kv].astype(np.float64)).astype(np.float32))
        for qi, q in enumerate((0, 1, 2)):
            mult = w.quality_mult[q]
            ls = np.array([0.5, 1.0, 1.0, 1.5])[:, None]
            want = mult * ls * sig
            got = tv.step[q][kv].astype(np.float64)
            assert np.allclose(got, want, rtol=2.0**-23, atol=0)
            assert np.array_equal(tv.inv_step[q][kv],
                                  (1.0 / got).astype(np.float32))
            f = tv.freq[q][kv].astype(np.int64)
            assert np.all(f.sum(axis=-1) == M) and f.min() >= 1
            c = counts[qi, kv]
            # every delta token is counted once: tokens minus anchors of each chunk
            n_delta = sum(tc - -(-tc // 10) for tc in (256, 256, 188))
            assert np.all(c.astype(np.int64).sum(axis=-1) == n_delta)
            for l in range(4):
                for ch in range(0, 96, 17):
                    assert np.array_equal(tv.freq[q][kv, l, ch], oracle_lib.normalize(c[l, ch]))
    assert len(t) == 80 + 8 * 2 * 4 * 96 + 3 * (8 + 128) * 2 * 4 * 96


def test_layer_group_steps_match_pages(oracle_lib):
    """Shallow / medium / deep layers of a 32-layer model use steps 0.5 / 1.0 /
    1.5 channel stds (constants printed on the CacheGen blog, section 1 and the
    section 2.1 pseudocode; the config's 1-10 / 11-20 / 21-32 split)."""
    g = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    w = synth.Workload("steps", layers=32, tokens=64, channels=8, seed=5, rho=0.8,
                       outlier_frac=0.0, chunk_tokens=64, group_tokens=g["group_tokens"],
                       layer_group_end=tuple(g["layer_group_end_32"]),
                       layer_step=tuple(g["layer_steps"]), qualities=(0, 1, 2))
    k, v = synth.gen_kv(w)
    t = oracle_lib.build_tables(oracle_lib.params_for(w), k, v)
    tv = oracle_lib.tables_view(t)
    sig = k.astype(np.float64).std(axis=1)
    for l in range(32):
        want = g["layer_steps"][0 if l < 10 else 1 if l < 20 else 2]
        for q, mult in enumerate(w.quality_mult):
            ratio = tv.step[q][0, l].astype(np.float64) / (sig[l] * mult)
            assert np.allclose(ratio, want, rtol=2.0**-22)


def test_nonfinite_input_is_rejected(oracle_lib):
    w = small_workload(layers=1, layer_group_end=(1,), layer_step=(0.5,), qualities=(0,))
    k, v = synth.gen_kv(w)
    v[0, 3, 3] = np.inf
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.build_tables(oracle_lib.params_for(w), k, v)
    assert e.value.code == -1


def test_bad_params_are_rejected(oracle_lib):
    k = np.zeros((2, 8, 4), np.float16)
    good = dict(layers=2, tokens=8, channels=4, chunk_tokens=8, group_tokens=4,
                layer_group_end=(2,), layer_step=(0.5,), quality_mask=1)
    oracle_lib.build_tables(oracle_lib.make_params(**good), k, k)
    for bad in (dict(layer_group_end=(1,)), dict(group_tokens=0), dict(group_tokens=9),
                dict(chunk_tokens=0), dict(quality_mask=0), dict(quality_mask=8),
                dict(layer_step=(-1.0,)), dict(layer_group_end=(2, 2), layer_step=(1, 1))):
        p = oracle_lib.make_params(**{**good, **bad})
        with pytest.raises(oracle_lib.OracleError):
            oracle_lib.build_tables(p, k, k)


def test_fnv_and_tables_id(oracle_lib):
    # FNV-1a-64 reference values: empty input is the offset basis; "a" and "foobar"
    # are the published test vectors of the FNV specification
    assert oracle_lib.fnv1a64(b"") == 0xcbf29ce484222325
    assert oracle_lib.fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert oracle_lib.fnv1a64(b"foobar") == 0x85944171f73967e8
    rng = np.random.default_rng(2)

    def fnv_of_digests(ds):
        return oracle_lib.fnv1a64(b"".join(x.to_bytes(8, "little") for x in ds))

    # the id is a three-level tree: 1 KiB leaves, middle digests over 256 leaves,
    # the id over the middle digests (sizes straddle every boundary)
    for n in (1, 1023, 1024, 1025, 262143, 262144, 262145, 600000):
        d = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        leaves = [oracle_lib.fnv1a64(d[i:i + 1024]) for i in range(0, n, 1024)]
        mids = [fnv_of_digests(leaves[j:j + 256]) for j in range(0, len(leaves), 256)]
        assert oracle_lib.tables_id(d) == fnv_of_digests(mids)
    # one changed byte anywhere changes the id
    d = bytearray(rng.integers(0, 256, 300000, dtype=np.uint8).tobytes())
    base = oracle_lib.tables_id(bytes(d))
    for pos in (0, 1023, 1024, 262143, 262144, 299999):
        e = bytearray(d)
        e[pos] ^= 1
        assert oracle_lib.tables_id(bytes(e)) != base
